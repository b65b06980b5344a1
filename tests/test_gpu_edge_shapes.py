"""GPU parity on shapes at the edges of what the library accepts, against the
oracle on every token: one expert with one K step in both GEMMs (and K ranges
split over waves that get no step); 300 experts (past the one-launch
prologues), top-16, three K steps, six GEMM2 units (not a multiple of four);
the tiled GEMMs with partial column bands and odd K steps; 1024 experts;
top-16 on the 64-token routing blocks with the tiled GEMMs.

Bit-exact: the per-token quantization, router ids, the permutation, the
re-quantization of every expanded row (NVFP4) or GEMM2's bf16 input
(W4A16).  Tolerance: the layer output as for the configured layers."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import (bf16_tensor_to_f64, check_layer_tolerance, gpu_weights,
                                  oracle_expert, oracle_weights, to_device_bf16)

pytestmark = pytest.mark.gpu

CASES = [(6, "nvfp4"), (6, "w4a16"), (7, "nvfp4"), (7, "atomic"), (7, "shared"), (8, "nvfp4"),
         (8, "w4a16"), (8, "shared"), (9, "nvfp4"), (11, "nvfp4"), (11, "atomic"), (11, "shared")]


@pytest.mark.parametrize("layer_id,mode", CASES)
def test_edge_shape(layer_id, mode):
    L = synth.LAYERS[layer_id]
    T, H, I, E, k = L.T, L.H, L.I, L.E, L.k
    shared = "sum" if mode == "shared" else None
    a16 = mode == "w4a16"
    det = mode != "atomic"
    print(f"layer {layer_id} ({L.name}) T={T} H={H} I={I} E={E} k={k} mode={mode}", flush=True)
    x, logits = synth.activations(layer_id), synth.router_logits(layer_id)
    layer = binding.MoeLayer(L.max_tokens, H, I, E, k, det, shared_expert=shared, w4a16=a16)
    layer.bind(gpu_weights(layer_id, n_experts=E + (1 if shared else 0)))
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    if not a16:
        xc = layer.read_buffer("XQ_CODES", torch.uint8, (T, H // 2)).cpu().numpy()
        xs = layer.read_buffer("XQ_SCALES", torch.uint8, (T, H // 16)).cpu().numpy()
        xg = layer.read_buffer("XQ_GSCALE", torch.float32, (T,)).cpu().numpy()
        oc, os_, og = oracle.quantize_rows(x)
        np.testing.assert_array_equal(xg, og)
        np.testing.assert_array_equal(xs, os_)
        np.testing.assert_array_equal(xc, oc)
    ids = layer.read_buffer("TOPK_IDS", torch.int32, (T, k)).cpu().numpy()
    w = layer.read_buffer("TOPK_W", torch.float32, (T, k)).cpu().numpy()
    oids, ow = oracle.router(logits, k)
    np.testing.assert_array_equal(ids, oids)
    np.testing.assert_allclose(w, ow, rtol=0, atol=2e-6)
    counts, offsets, perm, inv = oracle.permute(oids, E)
    np.testing.assert_array_equal(layer.read_buffer("COUNTS", torch.int32, (E,)).cpu().numpy(), counts)
    if det:
        np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (T * k,)).cpu().numpy(), perm)
        np.testing.assert_array_equal(layer.read_buffer("INV", torch.int32, (T * k,)).cpu().numpy(), inv)
    Rt = T * (k + (1 if shared else 0))
    act = layer.read_buffer("ACT", torch.float32, (Rt, I)).cpu().numpy()
    if a16:
        a2 = layer.read_buffer("A2_16", torch.int16, (Rt, I)).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(a2, oracle.f32_to_bf16(act))
    else:
        c, s, g = oracle.quantize_rows(act)
        np.testing.assert_array_equal(layer.read_buffer("A2_GSCALE", torch.float32, (Rt,)).cpu().numpy(), g)
        np.testing.assert_array_equal(layer.read_buffer("A2_SCALES", torch.uint8, (Rt, I // 16)).cpu().numpy(), s)
        np.testing.assert_array_equal(layer.read_buffer("A2_CODES", torch.uint8, (Rt, I // 2)).cpu().numpy(), c)
    toks = np.arange(T)
    routed = oracle_weights(layer_id, np.unique(oids))
    print(f"oracle: layer {layer_id} on {T} tokens", flush=True)
    if shared:
        sh = oracle.QuantWeights(np.array([E], np.int32), *(a[None] for a in oracle_expert(layer_id, E)))
        ref = oracle.moe_layer_shared(x, oids, ow, toks, H, I, routed, sh, shared, a16=a16)
    else:
        ref = oracle.moe_layer(x, oids, ow, toks, H, I, routed, a16=a16)
    check_layer_tolerance(bf16_tensor_to_f64(out), ref)
    layer.close()
