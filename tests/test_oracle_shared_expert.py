"""Pins of the oracle's shared-expert combination ([P3] Command-A-Plus
multi-stream page, Cohere2MoeSparseMoeBlock.forward: the routed and shared
outputs are added; the 'average' strategy halves the sum).  The shared expert
is an NVFP4 expert of the routed shape applied to every token with weight 1.

Each pin reaches the composed result by a different route: the brute-force
dense layer with one more always-selected expert, a shared expert equal to a
routed one, and an all-zero shared expert."""
import numpy as np
import pytest

import oracle
from nvfp4_token_quant_amd import synth
from tests.test_oracle_route_layer import _tiny_weights


def _setup():
    L = synth.LAYERS[1]
    x = synth.activations(1)
    ids, w = oracle.router(synth.router_logits(1), L.k)
    _, _, q13, q2 = _tiny_weights(E=L.E + 1)  # expert L.E is the shared one
    routed = oracle.QuantWeights(np.arange(L.E), *(a[:L.E] for a in q13), *(a[:L.E] for a in q2))
    shared = oracle.QuantWeights(np.array([L.E]), *(a[L.E:] for a in q13), *(a[L.E:] for a in q2))
    return L, x, ids, w, q13, q2, routed, shared


@pytest.mark.parametrize("strategy,c", [("sum", 1.0), ("average", 0.5)])
def test_shared_equals_dense_with_extra_expert(strategy, c):
    """Dense brute force over E + 1 experts, every token also selecting expert
    E with weight 1, all weights scaled by the strategy's factor."""
    L, x, ids, w, q13, q2, routed, shared = _setup()
    got = oracle.moe_layer_shared(x, ids, w, np.arange(L.T), L.H, L.I, routed, shared, strategy)
    ids_d = np.concatenate([ids, np.full((L.T, 1), L.E, np.int32)], axis=1)
    w_d = np.concatenate([w, np.ones((L.T, 1))], axis=1) * c
    dense = oracle.moe_layer_dense(x, ids_d, w_d, L.H, L.I, L.E + 1, *q13, *q2)
    np.testing.assert_allclose(got, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
    assert np.abs(got).max() > 0


def test_shared_copy_of_routed_expert():
    """Every token routed (k = 1, weight 1) to expert e0 and a shared expert
    holding e0's weights: both outputs are the same bits, so the sum is
    exactly twice the routed output and the average exactly equals it."""
    L, x, ids, w, q13, q2, routed, _ = _setup()
    e0 = 3
    ids1 = np.full((L.T, 1), e0, np.int32)
    w1 = np.ones((L.T, 1))
    copy = oracle.QuantWeights(np.array([e0]), *(a[e0:e0 + 1] for a in q13), *(a[e0:e0 + 1] for a in q2))
    r = oracle.moe_layer(x, ids1, w1, np.arange(L.T), L.H, L.I, routed)
    s = oracle.moe_layer_shared(x, ids1, w1, np.arange(L.T), L.H, L.I, routed, copy, "sum")
    a = oracle.moe_layer_shared(x, ids1, w1, np.arange(L.T), L.H, L.I, routed, copy, "average")
    np.testing.assert_array_equal(s, 2 * r)
    np.testing.assert_array_equal(a, r)


def test_zero_shared_expert():
    """A shared expert whose codes are all zero contributes exactly 0."""
    L, x, ids, w, q13, q2, routed, shared = _setup()
    zero = oracle.QuantWeights(shared.experts, np.zeros_like(shared.w13c), shared.w13s, shared.w13g,
                               np.zeros_like(shared.w2c), shared.w2s, shared.w2g)
    r = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, routed)
    np.testing.assert_array_equal(
        oracle.moe_layer_shared(x, ids, w, np.arange(L.T), L.H, L.I, routed, zero, "sum"), r)
    np.testing.assert_array_equal(
        oracle.moe_layer_shared(x, ids, w, np.arange(L.T), L.H, L.I, routed, zero, "average"), r / 2)


def test_shared_strategy_checked():
    L, x, ids, w, q13, q2, routed, shared = _setup()
    with pytest.raises(ValueError):
        oracle.moe_layer_shared(x, ids, w, np.arange(L.T), L.H, L.I, routed, shared, "max")
