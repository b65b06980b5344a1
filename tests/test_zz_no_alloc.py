"""GPU test of moe_nvfp4_forward_noalloc (the forward without a workspace,
its intermediates in the library's fixed device array) against
moe_nvfp4_forward on a workspace of the same configuration bound to the same
packed weights: bit-identical in the slot-ordered (deterministic) finalize,
within the layer tolerance in the atomic one.  Each case runs two calls in a
row, the second on a smaller batch, so the second forward runs over the
first one's leftovers in the shared array.  Forwards too large for the array
are refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import bf16_tensor_to_f64, check_layer_tolerance, gpu_weights, to_device_bf16

pytestmark = pytest.mark.gpu


def _inputs(layer_id, T):
    x = to_device_bf16(synth.activations(layer_id, T))
    logits = torch.from_numpy(synth.router_logits(layer_id, T)).cuda()
    return x, logits


@pytest.mark.parametrize("layer_id,Ts,deterministic,shared", [
    (2, (64, 13), True, None),       # decode-shaped: decode prologue, stream GEMMs
    (2, (300, 200), True, None),     # three-kernel and small-batch prologues
    (1, (256, 16), True, "average"),  # tiled GEMMs, then stream GEMMs; shared expert
    (2, (64, 7), False, None),       # atomic finalize
    (7, (33, 5), True, "sum"),       # 300 experts, top-16: three-kernel and one-block prologues
    (5, (7, 1), True, None),         # the large layer at a few tokens (7168-wide rows)
])
def test_noalloc_matches_workspace_forward(layer_id, Ts, deterministic, shared):
    L = synth.LAYERS[layer_id]
    print(f"noalloc layer {layer_id} T={Ts} deterministic={deterministic} shared={shared}", flush=True)
    wts = gpu_weights(layer_id, n_experts=L.E + (1 if shared else 0))
    cap = max(Ts)
    layer = binding.MoeLayer(cap, L.H, L.I, L.E, L.k, deterministic, shared_expert=shared)
    layer.bind(wts)
    cfg = binding.MoeConfig(cap, L.H, L.I, L.E, L.k, layer.cfg.flags)
    for T in Ts:
        x, logits = _inputs(layer_id, T)
        want = layer.forward(x, logits)
        got = torch.full_like(x, float("nan"))
        binding.forward_noalloc(cfg, wts, x, logits, got)
        torch.cuda.synchronize()
        if deterministic:
            assert torch.equal(got, want), f"T={T}"
        else:
            check_layer_tolerance(bf16_tensor_to_f64(got), bf16_tensor_to_f64(want))
    layer.close()


def test_noalloc_refuses_what_does_not_fit():
    """The large layer (H = 7168, E = 256, I = 2048, top-8) at 2048 tokens
    needs far more than the array; the call fails before any launch and the
    output stays untouched.  Static activation scales need a workspace."""
    L = synth.LAYERS[2]
    big = synth.LAYERS[5]
    wts = gpu_weights(2)
    x, logits = _inputs(2, 64)
    out = torch.zeros_like(x)
    # the decode weights stand in: the size check fails before any pointer is used
    cfg = binding.MoeConfig(8192, big.H, big.I, big.E, big.k, binding.MOE_DETERMINISTIC_FINALIZE)
    fake = binding.MoePacked(big.E, big.H, big.I, wts.w13.data_ptr(), wts.w13_gscale.data_ptr(),
                             wts.w2.data_ptr(), wts.w2_gscale.data_ptr())
    rc = binding.lib().moe_nvfp4_forward_noalloc(ctypes.byref(cfg), ctypes.byref(fake), x.data_ptr(),
                                                 logits.data_ptr(), 2048, out.data_ptr(), None)
    assert rc == 1
    msg = binding.lib().nvfp4_last_error().decode()
    assert "no-allocation forward holds" in msg, msg
    cfg = binding.MoeConfig(64, L.H, L.I, L.E, L.k, binding.MOE_STATIC_ACT_SCALES)
    with pytest.raises(binding.Nvfp4Error, match="MOE_STATIC_ACT_SCALES"):
        binding.forward_noalloc(cfg, wts, x, logits, out)
    cfg = binding.MoeConfig(32, L.H, L.I, L.E, L.k, binding.MOE_DETERMINISTIC_FINALIZE)
    with pytest.raises(binding.Nvfp4Error) as ei:
        binding.forward_noalloc(cfg, wts, x, logits, out)
    assert ei.value.status == "NVFP4_ERR_TOO_MANY_TOKENS"
    torch.cuda.synchronize()
    assert not out.any()
