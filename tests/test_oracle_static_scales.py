"""Pins of the oracle's static activation scales: the per-tensor input-scale
contract that per-token scaling replaces ([P1] sglang PR #28354 summary,
"Feature and motivation"; the static fc2_input_scale of "Source snippets").
The block recipe is the per-token one with the global scale given instead of
2688 / amax, so values beyond the given range saturate."""
import numpy as np
import pytest

import oracle
from nvfp4_token_quant_amd import synth
from tests.test_oracle_route_layer import _tiny_weights


def test_static_scale_saturates_block_and_codes():
    """Hand-derived: with g = 2688 a block holding 1000 needs a scale of
    1000 * 2688 / 6 = 448000, which saturates to the largest E4M3 value 448
    (0x7E); then r = 2688 / 448 = 6, and 1000 * 6 saturates to the largest
    E2M1 magnitude 6 (code 7) while 0.5 -> 3 (code 5), -0.25 -> -1.5 (code
    0xB), 0 -> 0.  Dequantized: 6 * 448 / 2688 = 1.0, 0.5, -0.25, 0."""
    x = np.zeros((1, 16), np.float32)
    x[0, :4] = [1000.0, 0.5, -0.25, 0.0]
    codes, S = oracle.quantize_rows_given_g(x, 2688.0)
    assert S[0, 0] == 0x7E
    nib = [(codes[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(4)]
    assert nib == [0x7, 0x5, 0xB, 0x0]
    deq = oracle.dequantize(codes, S, np.float32(2688.0))
    np.testing.assert_array_equal(deq[0, :4], [1.0, 0.5, -0.25, 0.0])


def _mini_layer(T, k, seed):
    """A small layer whose every x row has amax exactly 1.0 (so the per-row
    global scale of x is 2688 on every row)."""
    rng = np.random.default_rng(seed)
    H, I, E = 64, 32, 3
    x = rng.uniform(-1, 1, (T, H)).astype(np.float32)
    x[:, 0] = 1.0
    xb = synth.bf16_bits(x)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.1).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    q13, q2 = oracle.quantize_groups(w13), oracle.quantize_groups(w2)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T)
    qw = oracle.QuantWeights(np.arange(E), *q13, *q2)
    return xb, ids, w, qw, q13, q2, H, I, E


def test_static_scales_equal_per_row_scales_when_they_coincide():
    """One token routed to one expert: static scales equal to that row's own
    per-row scales (2688 for x, the dynamic g2 of the act row) give exactly the
    dynamic result; a different static g_a does not (a power-of-two factor
    would not show: it scales every block scale exactly and leaves the codes
    and the dequantized values as they are, hence 0.7)."""
    xb, ids, w, qw, *_, H, I, E = _mini_layer(T=1, k=1, seed=3)
    w = np.ones((1, 1))
    dyn, dbg = oracle.moe_layer(xb, ids, w, np.arange(1), H, I, qw, debug=True)
    g2 = float(dbg["g2"][0, 0])
    xc, xs, xg = oracle.quantize_rows(xb)
    assert xg[0] == np.float32(2688.0)
    stat = oracle.moe_layer(xb, ids, w, np.arange(1), H, I, qw, static_scales=(2688.0, g2))
    np.testing.assert_array_equal(stat, dyn)
    other = oracle.moe_layer(xb, ids, w, np.arange(1), H, I, qw, static_scales=(2688.0, 0.7 * g2))
    assert not np.array_equal(other, dyn)


def test_static_x_scale_equal_per_row_for_unit_amax_rows():
    """Every x row has amax 1.0, so a static g_x = 2688 quantizes x exactly as
    the per-token scales do: with the same static g_a on both sides the
    outputs are equal."""
    xb, ids, w, qw, *_, H, I, E = _mini_layer(T=6, k=2, seed=5)
    toks = np.arange(6)
    _, dbg = oracle.moe_layer(xb, ids, w, toks, H, I, qw, debug=True)
    ga = float(np.median(dbg["g2"]))
    a = oracle.moe_layer(xb, ids, w, toks, H, I, qw, static_scales=(2688.0, ga))
    # a non-positive component keeps the per-row scales: x per token, act static
    b = oracle.moe_layer(xb, ids, w, toks, H, I, qw, static_scales=(0.0, ga))
    np.testing.assert_array_equal(a, b)
    d = oracle.moe_layer(xb, ids, w, toks, H, I, qw, static_scales=(0.7 * 2688.0, ga))
    assert not np.array_equal(a, d)   # the static g_x is really used
    c, _ = oracle.moe_layer(xb, ids, w, toks, H, I, qw, debug=True)
    assert not np.array_equal(a, c)   # the static g_a is really used


@pytest.mark.parametrize("ga_factor", [1.0, 3.7])
def test_static_layer_equals_dense_bruteforce(ga_factor):
    """The tiny layer with static scales (g_x from the batch amax, g_a from
    the largest act value, or 3.7x larger so that GEMM2's largest inputs
    saturate): the compact layer equals the every-expert-on-every-token
    loop."""
    L = synth.LAYERS[1]
    x = synth.activations(1)
    ids, w = oracle.router(synth.router_logits(1), L.k)
    _, _, q13, q2 = _tiny_weights()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    _, dbg = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, debug=True)
    gx = float(oracle.global_scale(synth.bf16_to_f32(x)))
    ga = float(oracle.global_scale(dbg["act"])) * ga_factor
    out = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, static_scales=(gx, ga))
    dense = oracle.moe_layer_dense(x, ids, w, L.H, L.I, L.E, *q13, *q2, static_scales=(gx, ga))
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
    assert np.all(np.isfinite(out))
