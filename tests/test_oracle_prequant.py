"""Pins of the oracle's layer for activations handed over already quantized
([P1] sglang PR #28354 summary, "Implementation breakdown" item 2: the
runner is given FP4 codes, block scales and the per-token scale, and the
expert GEMMs consume them as they are)."""
import numpy as np
import pytest

import oracle
from tests import npref
from tests.test_oracle_static_scales import _mini_layer


def _numpy_layer(xh, ids, w, q13, q2, H, I, static_ga=None):
    """The layer restated in numpy from dequantized activation rows xh:
    weights dequantized through lookup tables, the GEMMs as float64 matmuls,
    the SwiGLU in float64 rounded to binary32, the GEMM2 input re-quantized
    by the oracle's row quantizer (pinned on its own) and dequantized by
    tables, the weighted sum over the slots."""
    w13 = npref.dequant(q13[0], q13[1], q13[2][:, None], g_per_row=True)
    w2 = npref.dequant(q2[0], q2[1], q2[2][:, None], g_per_row=True)
    T, k = ids.shape
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            h = w13[e] @ xh[t]
            z = h[:I]
            act = (z / (1.0 + np.exp(-z)) * h[I:]).astype(np.float32)[None]
            if static_ga is None:
                c2, s2, g2 = oracle.quantize_rows(act)
            else:
                c2, s2 = oracle.quantize_rows_given_g(act, static_ga)
                g2 = np.full(1, static_ga, np.float32)
            ah = npref.dequant(c2, s2, g2)[0]
            out[t] += w[t, j] * (w2[e] @ ah)
    return out


@pytest.mark.parametrize("T,k,seed", [(5, 2, 11), (9, 3, 12)])
def test_prequantized_layer_equals_layer_on_x(T, k, seed):
    """Codes, scales and scales of x from the oracle's own per-token Q give
    the layer on x exactly: the pre-quantized entry replaces only step 1."""
    xb, ids, w, qw, *_, H, I, E = _mini_layer(T, k, seed)
    tokens = np.arange(T)
    ref = oracle.moe_layer(xb, ids, w, tokens, H, I, qw)
    xc, xs, xg = oracle.quantize_rows(xb)
    got = oracle.moe_layer_quantized(xc, xs, xg, ids, w, tokens, H, I, qw)
    np.testing.assert_array_equal(got, ref)
    # and with a static GEMM2-input scale
    ref_s = oracle.moe_layer(xb, ids, w, tokens, H, I, qw, static_scales=(float(xg[0]), 3.5))
    got_s = oracle.moe_layer_quantized(xc, xs, xg, ids, w, tokens, H, I, qw, static_ga=3.5)
    np.testing.assert_array_equal(got_s, ref_s)


@pytest.mark.parametrize("static_ga", [None, 40.0])
def test_prequantized_layer_arbitrary_codes_against_numpy(static_ga):
    """Codes no bf16 row quantizes to (every nibble, the negative zero
    included; every finite scale byte; global scales over six decades) against
    the layer restated in numpy on their table-dequantized values."""
    rng = np.random.default_rng(5)
    T, k = 6, 2
    xb, ids, w, qw, q13, q2, H, I, E = _mini_layer(T, k, 21)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    xc = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    xs = rng.integers(0, 0x7F, (T, H // 16), dtype=np.uint8)  # 0x7F is NaN: excluded
    xg = (10.0 ** rng.uniform(0, 6, T)).astype(np.float32)
    xh = npref.dequant(xc, xs, xg)
    ref = _numpy_layer(xh, ids, w, q13, q2, H, I, static_ga)
    got = oracle.moe_layer_quantized(xc, xs, xg, ids, w, np.arange(T), H, I, qw, static_ga=static_ga)
    scale = np.abs(ref).max()
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12 * scale)


def test_prequantized_zero_codes_give_zero():
    """Rows whose codes are all +0 / -0 are zero whatever their scales: h,
    the SwiGLU output and the layer output are exactly zero (the all-zero act
    row re-quantizes to zero codes with global scale 1)."""
    T, k = 3, 2
    xb, ids, w, qw, *_, H, I, E = _mini_layer(T, k, 31)
    xc = np.zeros((T, H // 2), np.uint8)
    xc[1] = 0x88  # negative zeros
    xs = np.full((T, H // 16), 0x50, np.uint8)
    xg = np.full(T, 7.0, np.float32)
    got = oracle.moe_layer_quantized(xc, xs, xg, ids, w, np.arange(T), H, I, qw)
    assert np.all(got == 0.0)


def test_prequantized_missing_expert_raises():
    T, k = 2, 2
    xb, ids, w, qw, *_, H, I, E = _mini_layer(T, k, 41)
    xc, xs, xg = oracle.quantize_rows(xb)
    keep = qw.experts != ids[0, 0]
    qsub = oracle.QuantWeights(qw.experts[keep], qw.w13c[keep], qw.w13s[keep], qw.w13g[keep],
                               qw.w2c[keep], qw.w2s[keep], qw.w2g[keep])
    with pytest.raises(ValueError):
        oracle.moe_layer_quantized(xc, xs, xg, ids, w, np.arange(T), H, I, qsub)
