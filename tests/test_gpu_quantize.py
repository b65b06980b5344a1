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
def test_quantize_layer_full_size_sampled():
    """The quantize-only workload [16384, 7168] at full size: sampled rows
    bit-exact, plus properties on every row."""
    L = synth.LAYERS[4]
    x = synth.activations(4)
    print(f"quantize layer {L.T}x{L.H}", flush=True)
    c, s, g = _gpu_quant(x)
    rng = np.random.default_rng(0)
    xf = synth.bf16_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    zero = np.flatnonzero(amax == 0)
    big = np.argsort(amax)[-4:]
    sample = np.unique(np.concatenate([zero[:20], big, rng.choice(L.T, 300, replace=False),
                                       [0, L.T - 1]]))
    oc, os_, og = oracle.quantize_rows(x[sample])
    np.testing.assert_array_equal(c[sample], oc)
    np.testing.assert_array_equal(s[sample], os_)
    np.testing.assert_array_equal(g[sample], og)
    # every row: zero rows -> g 1, scales 0, codes 0; else the row-max block has 448
    assert np.all(g[zero] == 1.0) and not s[zero].any() and not c[zero].any()
    nz = np.flatnonzero(amax > 0)
    top_block = np.argmax(np.abs(xf[nz]), axis=1) // 16
    assert np.all(s[nz, top_block] == 0x7E)
    np.testing.assert_array_equal(g[nz], (np.float32(2688.0) / amax[nz]).astype(np.float32))


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
