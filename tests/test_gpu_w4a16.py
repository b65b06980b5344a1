"""GPU parity of the W4A16 mode (bf16 activations, NVFP4 weights) against the
oracle's a16 layer: x itself feeds GEMM1, the SwiGLU output rounded to bf16
(nearest even) feeds GEMM2; every batch size takes the tiled GEMMs (bf16
MFMA, weights dequantized exactly to bf16).

Bit-exact: router ids and the permutation, and GEMM2's bf16 input against the
bf16 rounding (the oracle's encoder) of the GPU's own SwiGLU output, on every
expanded row.  Tolerance: the layer output as for the NVFP4 layer, on every
token, or for the prefill and large layers on the tokens covering every
active expert's first and last expanded row (every tile shape)."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import (bf16_tensor_to_f64, check_layer_tolerance, covering_tokens,
                                  gpu_weights, oracle_expert, oracle_weights, to_device_bf16)

pytestmark = pytest.mark.gpu

_WEIGHTS = {}


def _weights(layer_id, n_experts):
    key = (layer_id, n_experts)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        torch.cuda.empty_cache()
        _WEIGHTS[key] = gpu_weights(layer_id, n_experts=n_experts)
    return _WEIGHTS[key]


def _check(layer_id, T, deterministic=True, shared=None, tokens=None, max_tokens=None):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} T={T} w4a16 deterministic={deterministic} shared={shared}", flush=True)
    x, logits = synth.activations(layer_id, T), synth.router_logits(layer_id, T)
    layer = binding.MoeLayer(max_tokens or max(T, L.max_tokens), L.H, L.I, L.E, L.k, deterministic,
                             shared_expert=shared, w4a16=True)
    layer.bind(_weights(layer_id, L.E + (1 if shared else 0)))
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ids = layer.read_buffer("TOPK_IDS", torch.int32, (T, L.k)).cpu().numpy()
    oids, ow = oracle.router(logits, L.k)
    np.testing.assert_array_equal(ids, oids)
    counts, offsets, perm, inv = oracle.permute(oids, L.E)
    if deterministic:
        np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (T * L.k,)).cpu().numpy(), perm)
    Rt = T * (L.k + (1 if shared else 0))
    act = layer.read_buffer("ACT", torch.float32, (Rt, L.I)).cpu().numpy()
    a16 = layer.read_buffer("A2_16", torch.int16, (Rt, L.I)).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(a16, oracle.f32_to_bf16(act))
    if isinstance(tokens, str):
        tokens, present, covered = covering_tokens(oids, L.E)
        assert present <= covered
    toks = np.arange(T) if tokens is None else tokens
    routed = oracle_weights(layer_id, np.unique(oids[toks]))
    if shared:
        sh = oracle.QuantWeights(np.array([L.E], np.int32), *(a[None] for a in oracle_expert(layer_id, L.E)))
        ref = oracle.moe_layer_shared(x, oids, ow, toks, L.H, L.I, routed, sh, shared, a16=True)
    else:
        ref = oracle.moe_layer(x, oids, ow, toks, L.H, L.I, routed, a16=True)
    check_layer_tolerance(bf16_tensor_to_f64(out)[toks], ref)
    layer.close()


@pytest.mark.parametrize("T,deterministic", [(16, True), (16, False), (256, True)])
def test_w4a16_tiny(T, deterministic):
    _check(1, T, deterministic, max_tokens=256)


@pytest.mark.parametrize("T", [1, 64])
def test_w4a16_decode(T):
    _check(2, T)


@pytest.mark.timeout(900)
def test_w4a16_prefill():
    """Prefill-shaped layer: GEMM2's bf16 input on every row, the layer on
    the tokens covering every expert's first and last expanded row."""
    _check(3, 4096, tokens="covering")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("T", [1, 7, 2048])
def test_w4a16_large(T):
    _check(5, T, tokens=None if T <= 7 else "covering")


def test_w4a16_with_shared_expert():
    _check(2, 64, shared="average")
