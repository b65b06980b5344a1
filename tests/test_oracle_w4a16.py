"""Pins of the oracle's W4A16 mode (bf16 activations, NVFP4 weights; the
variant the pages only name, as a related PR title on [P3], read here as
bf16 activations that skip both activation quantizations): x itself (bf16) is GEMM1's input, the SwiGLU
output rounded to bf16 (round to nearest, ties to even) is GEMM2's input, the
weights are dequantized NVFP4 with their per-expert global scales.

* the bf16 rounding against torch's float32 -> bfloat16 cast (a library),
  over random values across the exponent range, every tie pattern, the
  overflow edge, subnormals, signed zeros, infinities and NaN;
* the layer against an independent numpy / scipy / torch computation of the
  same formula (matmuls on LUT-dequantized weights);
* the layer against the brute-force dense loop (every expert on every token);
* on inputs that NVFP4 represents exactly (the lossless case), the W4A16
  GEMM1 input is the W4A4 one, so the SwiGLU outputs agree bit for bit."""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from nvfp4_token_quant_amd import synth
from tests import npref
from tests.test_oracle_quant import _fp4_exact_rows
from tests.test_oracle_route_layer import _tiny_weights


def _torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(11)
    vals = [np.clip(rng.standard_normal(20000) * 2.0 ** rng.integers(-140, 120, 20000),
                    -3.0e38, 3.0e38).astype(np.float32)]
    # every tie: kept part even / odd, dropped bits exactly 0x8000, and their neighbours
    kept = rng.integers(0, 1 << 16, 4000, dtype=np.uint32)
    for dropped in (0x8000, 0x7fff, 0x8001, 0x0000, 0xffff):
        vals.append(((kept << 16) | dropped).view(np.float32))
    specials = np.array([0x7f7fffff, 0x7f7f8000, 0x7f7f7fff, 0xff7fffff, 0x00000001, 0x00008000,
                         0x00018000, 0x807fffff, 0x00000000, 0x80000000, 0x7f800000, 0xff800000],
                        np.uint32).view(np.float32)
    vals.append(specials)
    x = np.concatenate(vals).astype(np.float32)
    finite = np.isfinite(x)
    got = oracle.f32_to_bf16(x)
    np.testing.assert_array_equal(got[finite], _torch_bf16_bits(x[finite]))
    # infinities stay infinities; overflow of the largest finite values rounds to them
    assert oracle.f32_to_bf16(np.array([np.inf, -np.inf], np.float32)).tolist() == [0x7f80, 0xff80]
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7f80) == 0x7f80 and (nan & 0x7f) != 0


def _layer():
    L = synth.LAYERS[1]
    x = synth.activations(1)
    ids, w = oracle.router(synth.router_logits(1), L.k)
    _, _, q13, q2 = _tiny_weights()
    return L, x, ids, w, q13, q2


def test_w4a16_against_numpy():
    L, x, ids, w, q13, q2 = _layer()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    got = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, a16=True)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    W13 = npref.dequant(q13[0], q13[1], q13[2][:, None, None], g_per_row=False)
    W2 = npref.dequant(q2[0], q2[1], q2[2][:, None, None], g_per_row=False)
    ref = np.zeros((L.T, L.H))
    for t in range(L.T):
        for j in range(L.k):
            e = ids[t, j]
            h = W13[e] @ xf[t]
            gate, up = h[:L.I], h[L.I:]
            act = (gate * expit(gate) * up).astype(np.float32)
            a16 = torch.from_numpy(act).to(torch.bfloat16).to(torch.float64).numpy()
            ref[t] += w[t, j] * (W2[e] @ a16)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-9 * np.abs(ref).max())
    # and it is not the W4A4 layer
    assert np.abs(got - oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw)).max() > 0


def test_w4a16_equals_dense_bruteforce():
    L, x, ids, w, q13, q2 = _layer()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    got = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, a16=True)
    dense = oracle.moe_layer_dense(x, ids, w, L.H, L.I, L.E, *q13, *q2, a16=True)
    np.testing.assert_allclose(got, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


def test_lossless_inputs_give_the_w4a4_swiglu():
    """x on the NVFP4 grid: Q(x) dequantizes to x, so GEMM1 sees the same
    input in both modes and the SwiGLU outputs are the same bits."""
    L, _, ids, w, q13, q2 = _layer()
    rng = np.random.default_rng(5)
    x = synth.bf16_bits(_fp4_exact_rows(rng, L.T, L.H))
    assert np.array_equal(synth.bf16_to_f32(x), _fp4_exact_rows(np.random.default_rng(5), L.T, L.H))
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    _, d4 = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, debug=True)
    _, d16 = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw, debug=True, a16=True)
    np.testing.assert_array_equal(d16["act"], d4["act"])
    assert np.abs(d16["y"] - d4["y"]).max() > 0   # GEMM2 inputs differ (bf16 vs NVFP4)
