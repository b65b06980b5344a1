"""GPU parity of the layer with static activation scales (the per-tensor
input-scale contract that per-token scaling replaces, [P1] sglang PR #28354
summary, "Feature and motivation"; the static fc2_input_scale of "Source
snippets"): x quantized with one given g_x, the SwiGLU output with one given
g_a, the same block recipe (values beyond range saturate).

Bit-exact: the quantized x (codes, scales, g), router and permutation, the
re-quantized activation against the oracle's quantizer with g_a applied to the
GPU's own act; tolerance: the layer output against the oracle's static layer.
g_a is 3.7x the calibrated value, so the largest GEMM2 inputs saturate.
Batch sizes cover the decode-sized, small-batch and three-kernel prologues and
both re-quantization paths (fused into the GEMM2 stream kernel, and the
separate kernel before the tiled GEMM2), up to the prefill-shaped layer at full
size (T = 4096; its layer output on the tokens covering every expert's first
and last expanded row), and the large layer at one and seven tokens (rows of
7168, GEMM2's K of 2048)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import (bf16_tensor_to_f64, check_layer_tolerance, covering_tokens, gpu_weights,
                                  oracle_weights, to_device_bf16)

pytestmark = pytest.mark.gpu

_W = {}


def _weights(layer_id):
    if layer_id not in _W:
        _W.clear()
        torch.cuda.empty_cache()
        _W[layer_id] = gpu_weights(layer_id)
    return _W[layer_id]


def _scales(layer_id, x, ids, w, T):
    """g_x from the whole batch's amax; g_a from the oracle's act amax over a
    few tokens (calibration), times 3.7."""
    L = synth.LAYERS[layer_id]
    gx = float(oracle.global_scale(synth.bf16_to_f32(x)))
    toks = np.arange(min(T, 4))
    qw = oracle_weights(layer_id, np.unique(ids[toks]))
    _, dbg = oracle.moe_layer(x, ids, w, toks, L.H, L.I, qw, debug=True)
    ga = float(oracle.global_scale(dbg["act"])) * 3.7
    return gx, ga


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer_id,T", [(1, 16), (1, 256), (2, 64), (2, 301), (3, 4096), (5, 1), (5, 7)])
def test_static_scales_parity(layer_id, T):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} T={T} static scales", flush=True)
    x, logits = synth.activations(layer_id, T), synth.router_logits(layer_id, T)
    ids, w = oracle.router(logits, L.k)
    gx, ga = _scales(layer_id, x, ids, w, T)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True, static_act_scales=True)
    layer.bind(_weights(layer_id))
    layer.set_act_scales(torch.tensor([gx, ga], dtype=torch.float32, device="cuda"))
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    H, I, k, R = L.H, L.I, L.k, T * L.k
    # quantized x with the static g_x
    xc = layer.read_buffer("XQ_CODES", torch.uint8, (T, H // 2)).cpu().numpy()
    xs = layer.read_buffer("XQ_SCALES", torch.uint8, (T, H // 16)).cpu().numpy()
    xg = layer.read_buffer("XQ_GSCALE", torch.float32, (T,)).cpu().numpy()
    oc, os_ = oracle.quantize_rows_given_g(synth.bf16_to_f32(x), gx)
    np.testing.assert_array_equal(xg, np.float32(gx))
    np.testing.assert_array_equal(xs, os_)
    np.testing.assert_array_equal(xc, oc)
    # router and permutation are untouched by the scales
    np.testing.assert_array_equal(layer.read_buffer("TOPK_IDS", torch.int32, (T, k)).cpu().numpy(), ids)
    _, _, perm, _ = oracle.permute(ids, L.E)
    np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (R,)).cpu().numpy(), perm)
    # re-quantization with the static g_a, on the GPU's own act
    act = layer.read_buffer("ACT", torch.float32, (R, I)).cpu().numpy()
    a2c = layer.read_buffer("A2_CODES", torch.uint8, (R, I // 2)).cpu().numpy()
    a2s = layer.read_buffer("A2_SCALES", torch.uint8, (R, I // 16)).cpu().numpy()
    a2g = layer.read_buffer("A2_GSCALE", torch.float32, (R,)).cpu().numpy()
    c2, s2 = oracle.quantize_rows_given_g(act, ga)
    np.testing.assert_array_equal(a2g, np.float32(ga))
    np.testing.assert_array_equal(a2s, s2)
    np.testing.assert_array_equal(a2c, c2)
    assert (a2s == 0x7E).any(), "the 3.7x g_a should saturate some block scales"
    # the layer against the oracle's static layer
    if T <= 64:
        toks = np.arange(T)
    elif layer_id == 3:
        toks, present, covered = covering_tokens(ids, L.E)
        assert present <= covered
    else:
        toks = np.array([0, 1, T // 2, T - 1])
    qw = oracle_weights(layer_id, np.unique(ids[toks]))
    ref = oracle.moe_layer(x, ids, w, toks, H, I, qw, static_scales=(gx, ga))
    check_layer_tolerance(bf16_tensor_to_f64(out)[toks], ref)
    layer.close()


def test_static_scales_update_in_place_under_graph():
    """A captured forward picks up new static scales set in place: its replay
    equals an eager forward with the new values, bit for bit."""
    L = synth.LAYERS[2]
    x = to_device_bf16(synth.activations(2))
    logits = torch.from_numpy(synth.router_logits(2)).cuda()
    layer = binding.MoeLayer(L.T, L.H, L.I, L.E, L.k, True, static_act_scales=True)
    layer.bind(_weights(2))
    scales = torch.tensor([300.0, 2000.0], dtype=torch.float32, device="cuda")
    layer.set_act_scales(scales)
    out = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward_into(x, logits, out)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            layer.forward_into(x, logits, out)
    torch.cuda.synchronize()
    first = out.clone()
    layer.set_act_scales(torch.tensor([450.0, 1300.0], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        eager = layer.forward(x, logits)
        torch.cuda.synchronize()
        assert torch.equal(replayed, eager)
    assert not torch.equal(replayed, first)
    layer.close()


def test_static_scales_errors():
    L = synth.LAYERS[1]
    x = to_device_bf16(synth.activations(1))
    logits = torch.from_numpy(synth.router_logits(1)).cuda()
    layer = binding.MoeLayer(L.T, L.H, L.I, L.E, L.k, True, static_act_scales=True)
    layer.bind(_weights(1))
    with pytest.raises(RuntimeError, match="static activation scales not set"):
        layer.forward(x, logits)
    layer.close()
    plain = binding.MoeLayer(L.T, L.H, L.I, L.E, L.k, True)
    with pytest.raises(RuntimeError, match="MOE_STATIC_ACT_SCALES"):
        plain.set_act_scales(torch.ones(2, dtype=torch.float32, device="cuda"))
    plain.close()
