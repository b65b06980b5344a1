"""GPU parity of the quantizers against the CPU oracle (bit-exact).

Per-token quantization (nvfp4_quantize_per_token) and the per-expert weight
quantizer (nvfp4_quantize_experts) must reproduce the oracle's codes, E4M3
scale bytes and binary32 global scales exactly: both take every decision in
binary32 with the same operation order.
"""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import to_device_bf16

pytestmark = pytest.mark.gpu


def _gpu_quant(x_bits, ld=None):
    x = to_device_bf16(x_bits)
    if ld is not None:
        big = torch.zeros((x.shape[0], ld), dtype=torch.bfloat16, device="cuda")
        big[:, : x.shape[1]] = x
        x = big[:, : x_bits.shape[1]]
    c, s, g = binding.quantize_per_token(x)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), g.cpu().numpy()


def _rows(rng, rows, cols):
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    if rows > 2:
        x[1] = 0.0                              # all-zero row
        x[2] *= np.float32(1e-39)               # bf16 denormals: global scale clamps
    if rows > 4:
        x[3] *= np.float32(1e30)
        x[4, ::3] = 0.0
    return synth.bf16_bits(x)


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 256), (67, 2048), (130, 7168), (5, 8192),
                                       (9, 8208), (2, 16384), (257, 48)])
def test_per_token_bit_exact(rows, cols):
    print(f"quantize rows={rows} cols={cols}", flush=True)
    x = _rows(np.random.default_rng(rows * 7 + cols), rows, cols)
    c, s, g = _gpu_quant(x)
    oc, os_, og = oracle.quantize_rows(x)
    np.testing.assert_array_equal(g.view(np.uint32), og.view(np.uint32))
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)


def test_per_token_strided_rows():
    x = _rows(np.random.default_rng(5), 33, 512)
    c, s, g = _gpu_quant(x, ld=520)
    oc, os_, og = oracle.quantize_rows(x)
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(g, og)


def test_grid_midpoints_and_ties():
    """Values placed on E2M1 decision boundaries after scaling."""
    rng = np.random.default_rng(9)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    x = np.zeros((64, 64), np.float32)
    for r in range(64):
        x[r] = rng.choice(mids, 64) * rng.choice([-1, 1], 64) * np.float32(2.0 ** rng.integers(-8, 8))
        x[r, rng.integers(0, 64)] = np.float32(6.0 * 2.0 ** rng.integers(-8, 8))
    xb = synth.bf16_bits(x)
    c, s, g = _gpu_quant(xb)
    oc, os_, og = oracle.quantize_rows(xb)
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(g, og)


@pytest.mark.timeout(600)
def test_quantize_layer_full_size():
    """The quantize-only workload [16384, 7168] (Student-t(3) rows, every
    97th row zero, 4 rows x1e3) at full size: codes, scale bytes and global
    scales of every row bit-exact, plus the format's properties on every
    row."""
    L = synth.LAYERS[4]
    x = synth.activations(4)
    print(f"quantize layer {L.T}x{L.H}", flush=True)
    c, s, g = _gpu_quant(x)
    oc, os_, og = oracle.quantize_rows(x)
    np.testing.assert_array_equal(g.view(np.uint32), og.view(np.uint32))
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)
    xf = synth.bf16_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    zero = np.flatnonzero(amax == 0)
    assert len(zero) == len(range(0, L.T, 97))
    # zero rows -> g 1, scales 0, codes 0; else the row-max block has 448
    assert np.all(g[zero] == 1.0) and not s[zero].any() and not c[zero].any()
    nz = np.flatnonzero(amax > 0)
    top_block = np.argmax(np.abs(xf[nz]), axis=1) // 16
    assert np.all(s[nz, top_block] == 0x7E)
    np.testing.assert_array_equal(g[nz], (np.float32(2688.0) / amax[nz]).astype(np.float32))


def _finite_bf16_patterns():
    """Every finite bf16 bit pattern (both signs, zeros and subnormals
    included; the 256 inf / NaN patterns left out)."""
    b = np.arange(1 << 16, dtype=np.uint32)
    return b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _pack_blocks(blocks, cols=16384):
    """Rows of `cols` columns filled with 16-element blocks in the given
    order (sorted by block magnitude so that one row's blocks lie within a
    narrow range and keep nonzero E4M3 scales); each row's first block
    carries the row's largest block maximum."""
    nb = cols // 16
    order = np.argsort(np.abs(synth.bf16_to_f32(blocks)).max(axis=1), kind="stable")
    blocks = blocks[order]
    rows = (len(blocks) + nb - 1) // nb
    pad = rows * nb - len(blocks)
    if pad:
        blocks = np.concatenate([blocks, np.zeros((pad, 16), np.uint16)])
    out = blocks.reshape(rows, nb, 16)
    # move each row's largest block to the front (the order within a row does
    # not change any block's result, only which block holds the row max)
    mags = np.abs(synth.bf16_to_f32(out)).max(axis=2)
    top = mags.argmax(axis=1)
    r = np.arange(rows)
    first = out[r, 0].copy()
    out[r, 0] = out[r, top]
    out[r, top] = first
    return out.reshape(rows, cols)


def _encoder_sweep_rows():
    """Rows of the encoder sweep (see test_device_encoders_sweep)."""
    pats = _finite_bf16_patterns()
    vals = synth.bf16_to_f32(pats)
    posv = vals[vals > 0]                        # ascending
    cols = 16384
    nb = cols // 16
    rows = []
    # block scales: row max M in block 0, then every positive a <= M as the
    # maximum of one block [a, a/3, -a/7, 0, ...]
    for M in (2.0 ** -126, 2.0 ** -60, 1e-3, 1.0, 6.0, 448.0, 2688.0, 3e5, 2.0 ** 64, 2.0 ** 127):
        Mb = synth.bf16_to_f32(synth.bf16_bits(np.array([M], np.float32)))[0]
        a = posv[posv <= Mb]
        for i in range(0, len(a), nb - 1):
            ch = a[i:i + nb - 1]
            row = np.zeros((nb, 16), np.float32)
            row[0, 0] = Mb
            row[1:1 + len(ch), 0] = ch
            row[1:1 + len(ch), 1] = ch / 3
            row[1:1 + len(ch), 2] = -ch / 7
            rows.append(synth.bf16_bits(row).reshape(cols))
    x_scales = np.stack(rows)
    # element codes: element v (and -v) in a block of maximum B = 6 |v| / t
    # for t near each decision point; the blocks are sorted by B and packed
    # into rows, so each row's blocks keep full-precision E4M3 scales
    nz = pats[vals != 0]
    nzv = np.abs(vals[vals != 0])
    blocks = []
    for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        for f in (0.999, 1.0, 1.001):
            with np.errstate(over="ignore"):
                B = nzv * np.float32(6.0 / (t * f))
            ok = np.isfinite(B) & (B < 3.0e38)
            Bb = synth.bf16_bits(np.where(ok, B, 0).astype(np.float32))
            ok &= synth.bf16_to_f32(Bb) >= nzv
            blk = np.zeros((int(ok.sum()), 16), np.uint16)
            blk[:, 0] = Bb[ok]
            blk[:, 5] = nz[ok]
            blk[:, 9] = nz[ok] ^ 0x8000
            blocks.append(blk)
    x = np.concatenate([x_scales, _pack_blocks(np.concatenate(blocks), cols)])
    return x


@pytest.mark.timeout(600)
def test_device_encoders_sweep():
    """The device's E4M3 and E2M1 encoders, driven through
    nvfp4_quantize_per_token, against the oracle's encoders (written as
    searches over the formats' values), bit for bit:
      * block scales: every positive finite bf16 value as a block maximum,
        under row maxima from 2^-126 to 2^127 (so every block scale
        RN(RN(a * g) / 6) that a bf16 block can produce under those global
        scales, saturation at 448 and underflow to 0 included);
      * element codes: every finite bf16 value as a non-maximal element of a
        block whose maximum puts it near each E2M1 decision point (0.25,
        0.75, 1.25, 1.75, 2.5, 3.5, 5 after scaling) from both sides."""
    x = _encoder_sweep_rows()
    print(f"encoder sweep: {x.shape[0]} rows x {x.shape[1]}", flush=True)
    c, s, g = _gpu_quant(x)
    oc, os_, og = oracle.quantize_rows(x)
    np.testing.assert_array_equal(g.view(np.uint32), og.view(np.uint32))
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)
    # the sweep reaches saturated, zero and subnormal scale bytes, every code
    assert (s == 0x7E).any() and (s == 0).any() and ((s > 0) & (s < 8)).any()
    assert len(np.unique(np.concatenate([c & 15, c >> 4]))) == 16


def test_expert_quantizer_bit_exact():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(5, 96, 384)).astype(np.float32)
    w[2, 7, 9] = 3.0
    w[4] = 0.0
    c, s, g = binding.quantize_experts(torch.from_numpy(w).cuda())
    oc, os_, og = oracle.quantize_groups(w)
    np.testing.assert_array_equal(g.cpu().numpy(), og)
    np.testing.assert_array_equal(s.cpu().numpy(), os_)
    np.testing.assert_array_equal(c.cpu().numpy(), oc)


@pytest.mark.parametrize("layer_id,which,expert", [(1, 1, 0), (2, 1, 5), (2, 2, 127), (5, 2, 200)])
def test_synth_weights_match_oracle_generator(layer_id, which, expert):
    L = synth.LAYERS[layer_id]
    shape = synth.weight_shapes(layer_id)[which - 1]
    key = synth.weight_key(layer_id, which)
    got = binding.synth_weights(*key, expert, 1, shape, L.sigma)[0].cpu().numpy()
    want = oracle.synth_weights(*key, expert, shape, L.sigma)
    np.testing.assert_array_equal(got, want)
