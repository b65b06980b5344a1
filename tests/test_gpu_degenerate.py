"""Degenerate layers against the oracle: one expert with top-1 (every token
routed to it with weight 1), two experts with top-2 (every token takes both),
every token routed to one of several experts (the others receive none), and
the smallest dimensions the boundary accepts (H = 128: GEMM1 has a single K
step; I = 256: GEMM2 has two), each at batch sizes that take the stream and
the tiled GEMMs (ragged last tiles), in both finalize modes.

Inputs: x ~ N(0, 1) bf16, weights ~ N(0, 0.05), logits ~ N(0, 1) (plus a
bias that sends every token to one expert where stated), seeded.  Each side
quantizes the weights itself (the library's nvfp4_quantize_experts, the
oracle's Q); the codes are compared bit for bit before the layer is."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import bf16_tensor_to_f64, check_layer_tolerance, to_device_bf16

pytestmark = pytest.mark.gpu


def _case(E, k, H, I, T, seed, bias_expert=None, deterministic=True, max_tokens=None):
    print(f"E={E} k={k} H={H} I={I} T={T} bias={bias_expert} deterministic={deterministic}", flush=True)
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if bias_expert is not None:
        logits[:, bias_expert] += 50.0
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.05).astype(np.float32)
    # each side quantizes its own copy
    g13 = binding.quantize_experts(torch.from_numpy(w13).cuda())
    g2 = binding.quantize_experts(torch.from_numpy(w2).cuda())
    q13, q2 = oracle.quantize_groups(w13), oracle.quantize_groups(w2)
    for gpu, ref in zip(g13 + g2, q13 + q2):
        np.testing.assert_array_equal(gpu.cpu().numpy(), ref)
    layer = binding.MoeLayer(max_tokens or T, H, I, E, k, deterministic)
    layer.bind(binding.NvFp4Weights(*g13, *g2))
    out = layer.forward(to_device_bf16(x), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    ids, w = oracle.router(logits, k)
    np.testing.assert_array_equal(layer.read_buffer("TOPK_IDS", torch.int32, (T, k)).cpu().numpy(), ids)
    counts, offsets, perm, inv = oracle.permute(ids, E)
    np.testing.assert_array_equal(layer.read_buffer("COUNTS", torch.int32, (E,)).cpu().numpy(), counts)
    if deterministic:
        np.testing.assert_array_equal(layer.read_buffer("PERM", torch.int32, (T * k,)).cpu().numpy(), perm)
    qw = oracle.QuantWeights(np.arange(E), *q13, *q2)
    ref = oracle.moe_layer(x, ids, w, np.arange(T), H, I, qw)
    check_layer_tolerance(bf16_tensor_to_f64(out), ref)
    layer.close()
    return counts


@pytest.mark.parametrize("T", [1, 5, 64, 300])
def test_single_expert_top1(T):
    counts = _case(E=1, k=1, H=128, I=256, T=T, seed=10 + T)
    assert counts[0] == T


@pytest.mark.parametrize("T,deterministic", [(7, True), (200, True), (200, False)])
def test_two_experts_top2(T, deterministic):
    counts = _case(E=2, k=2, H=256, I=128, T=T, seed=20 + T, deterministic=deterministic)
    assert list(counts) == [T, T]


@pytest.mark.parametrize("T", [3, 130])
def test_all_tokens_to_one_expert(T):
    """Four experts, top-1, every token biased to expert 2: the other three
    receive no rows (no tiles, no work) and expert 2 takes all of them."""
    counts = _case(E=4, k=1, H=128, I=128, T=T, seed=30 + T, bias_expert=2, max_tokens=256)
    assert list(counts) == [0, 0, T, 0]
