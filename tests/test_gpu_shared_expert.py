"""GPU parity of the shared expert ([P3] Command-A-Plus multi-stream page,
Cohere2MoeSparseMoeBlock.forward: routed + shared, halved under 'average')
against the oracle's moe_layer_shared.  The shared expert is expert E of a
weight set of E + 1 experts (generated like the routed ones); the GPU runs
it as one more group of T expanded rows.

Bit-exact: the per-token quantization, router and permutation of the routed
part (unchanged by the shared expert), and the re-quantization of every
expanded row, the shared rows included.  Tolerance: the layer output as for
the routed layer."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import (bf16_tensor_to_f64, check_layer_tolerance, gpu_weights,
                                  oracle_expert, oracle_weights, to_device_bf16)

pytestmark = pytest.mark.gpu

_WEIGHTS = {}


def _weights(layer_id):
    if layer_id not in _WEIGHTS:
        _WEIGHTS.clear()
        torch.cuda.empty_cache()
        _WEIGHTS[layer_id] = gpu_weights(layer_id, n_experts=synth.LAYERS[layer_id].E + 1)
    return _WEIGHTS[layer_id]


def _layer(layer_id, strategy, deterministic=True, max_tokens=None):
    L = synth.LAYERS[layer_id]
    layer = binding.MoeLayer(max_tokens or L.max_tokens, L.H, L.I, L.E, L.k, deterministic,
                             shared_expert=strategy)
    layer.bind(_weights(layer_id))
    return layer


def _oracle(layer_id, x, ids, w, tokens, strategy):
    L = synth.LAYERS[layer_id]
    routed = oracle_weights(layer_id, np.unique(ids[tokens]))
    shared = oracle.QuantWeights(np.array([L.E], np.int32),
                                 *(a[None] for a in oracle_expert(layer_id, L.E)))
    return oracle.moe_layer_shared(x, ids, w, tokens, L.H, L.I, routed, shared, strategy)


def _check(layer_id, T, strategy, deterministic=True, max_tokens=None, tokens=None):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} T={T} shared={strategy} deterministic={deterministic}", flush=True)
    x, logits = synth.activations(layer_id, T), synth.router_logits(layer_id, T)
    layer = _layer(layer_id, strategy, deterministic, max_tokens)
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    # routed part of the integer path
    ids = layer.read_buffer("TOPK_IDS", torch.int32, (T, L.k)).cpu().numpy()
    oids, ow = oracle.router(logits, L.k)
    np.testing.assert_array_equal(ids, oids)
    counts, offsets, perm, inv = oracle.permute(oids, L.E)
    np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (T * L.k,)).cpu().numpy(), perm)
    # every expanded row's re-quantization, the T shared rows after the routed ones
    Rt, I = T * (L.k + 1), L.I
    rows = np.arange(Rt) if Rt <= 4096 else np.concatenate(
        [np.arange(0, T * L.k, 97), np.arange(T * L.k, Rt)])
    act = layer.read_buffer("ACT", torch.float32, (Rt, I)).cpu().numpy()[rows]
    c, s, g = oracle.quantize_rows(act)
    np.testing.assert_array_equal(layer.read_buffer("A2_GSCALE", torch.float32, (Rt,)).cpu().numpy()[rows], g)
    np.testing.assert_array_equal(layer.read_buffer("A2_SCALES", torch.uint8, (Rt, I // 16)).cpu().numpy()[rows], s)
    np.testing.assert_array_equal(layer.read_buffer("A2_CODES", torch.uint8, (Rt, I // 2)).cpu().numpy()[rows], c)
    toks = np.arange(T) if tokens is None else tokens
    ref = _oracle(layer_id, x, oids, ow, toks, strategy)
    rel = check_layer_tolerance(bf16_tensor_to_f64(out)[toks], ref)
    layer.close()
    return rel


@pytest.mark.parametrize("strategy", ["sum", "average"])
def test_shared_tiny(strategy):
    _check(1, 16, strategy)


@pytest.mark.parametrize("strategy,deterministic", [("sum", True), ("average", True), ("sum", False)])
def test_shared_decode_stream_path(strategy, deterministic):
    _check(2, 64, strategy, deterministic)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 7])
def test_shared_large_layer(T):
    """The large layer (rows of 7168, 257 expert weight sets) with its shared
    expert at one and seven tokens."""
    _check(5, T, "sum")


@pytest.mark.parametrize("T,deterministic", [(160, True), (256, False)])
def test_shared_tiled_path(T, deterministic):
    """The tiny layer at batch sizes that take the tiled GEMMs."""
    _check(1, T, "average", deterministic, max_tokens=T)


@pytest.mark.timeout(900)
def test_shared_prefill_sampled():
    rng = np.random.default_rng(2)
    _check(3, 4096, "sum", tokens=np.sort(rng.choice(4096, 32, replace=False)))


def test_shared_ragged_batches_and_weight_count():
    """T = 1 and 13 on a workspace sized for 64 (the shared expert's tile
    count follows T); weights without the shared expert are refused."""
    L = synth.LAYERS[2]
    x, logits = synth.activations(2), synth.router_logits(2)
    layer = _layer(2, "sum")
    full = bf16_tensor_to_f64(layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda()))
    for T in (1, 13):
        out = bf16_tensor_to_f64(layer.forward(to_device_bf16(x[:T]), torch.from_numpy(logits[:T]).cuda()))
        np.testing.assert_array_equal(out, full[:T])
    layer.close()
    wts = _weights(2)
    routed_only = wts.experts(0, L.E)
    layer = binding.MoeLayer(L.T, L.H, L.I, L.E, L.k, True, shared_expert="sum")
    with pytest.raises(binding.Nvfp4Error) as ei:
        layer.bind(routed_only)
    assert ei.value.status == "NVFP4_ERR_INVALID_ARG"
    layer.close()
