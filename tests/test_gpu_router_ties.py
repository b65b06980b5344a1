"""GPU parity of the router on tied logits, signed zeros included.

Logits drawn from {-0, +0, -1, 0.5, 1} tie constantly; -0.0 and +0.0 are
equal in a binary32 comparison, so every tie must go to the smaller expert
index with the slots in that order, exactly as the oracle's router decides.
Covered on the four prologue paths (one block routing every token for
T <= 64, with a whole wave per token up to 8 tokens and 16 lanes per token
above; the small-batch block for T <= 256; routing blocks of 64 tokens for
up to 256 experts and 8192 tokens, a last block of fewer tokens, down to
one, included; the three-kernel schedule past those) and with 1 to 16 keys
per lane (8 to 1024 experts): router ids and weights, the stable
expandInputRows permutation, and the layer output against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import (bf16_tensor_to_f64, check_layer_tolerance, gpu_weights,
                                  oracle_weights, to_device_bf16)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layer_id,T", [(1, 16), (1, 100), (1, 300), (1, 5), (2, 8), (2, 64), (10, 8),
                                        (10, 40), (9, 3), (2, 300), (10, 520), (7, 300), (11, 300), (11, 129)])
def test_router_ties_and_signed_zeros(layer_id, T):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} tied logits T={T}", flush=True)
    rng = np.random.default_rng(T)
    vals = np.array([-0.0, 0.0, -1.0, 0.5, 1.0], np.float32)
    logits = rng.choice(vals, size=(T, L.E)).astype(np.float32)
    logits[0] = -0.0
    logits[1] = 0.0
    logits[2, ::2] = -0.0
    x = synth.activations(layer_id, T)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True)
    layer.bind(gpu_weights(layer_id))
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ids = layer.read_buffer("TOPK_IDS", torch.int32, (T, L.k)).cpu().numpy()
    w = layer.read_buffer("TOPK_W", torch.float32, (T, L.k)).cpu().numpy()
    oids, ow = oracle.router(logits, L.k)
    np.testing.assert_array_equal(ids, oids)
    np.testing.assert_allclose(w, ow, rtol=0, atol=2e-6)
    counts, offsets, perm, inv = oracle.permute(oids, L.E)
    np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (T * L.k,)).cpu().numpy(), perm)
    np.testing.assert_array_equal(layer.read_buffer("INV", torch.int32, (T * L.k,)).cpu().numpy(), inv)
    ref = oracle.moe_layer(x, oids, ow, np.arange(T), L.H, L.I, oracle_weights(layer_id, np.unique(oids)))
    check_layer_tolerance(bf16_tensor_to_f64(out), ref)
    layer.close()
