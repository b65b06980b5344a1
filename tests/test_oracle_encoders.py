"""Pins of the oracle's E2M1 / E4M3 encoders and the Philox generator.

The oracle encodes by searching the format's values for the nearest one.
These tests check it against formulations that share none of that code:
  * E2M1: rounding to the binade's quantum with np.rint (ties to even), i.e.
    E2M1 treated as a tiny binary float format (OCP MX v1.0, FP4 E2M1);
  * E4M3: torch's float8_e4m3fn cast (library; OFP8 E4M3 "fn");
  * Philox4x64-10: the published known-answer vector and numpy's Philox.
"""
import numpy as np
import pytest

import oracle
from tests import npref


def _all_bf16_floats():
    b = np.arange(65536, dtype=np.uint32) << 16
    f = b.view(np.float32)
    return f[np.isfinite(f)]


def _e2m1_probe_values():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)
    pts = np.concatenate([mags, mids, np.array([6.5, 7.0, 8.0, 1e6], np.float32)])
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(-np.inf))])
    near = np.abs(near)
    rng = np.random.default_rng(1)
    rand = rng.uniform(0, 8, 20000).astype(np.float32)
    v = np.concatenate([near, rand, _all_bf16_floats()])
    v = v[np.abs(v) < 1e30]
    return np.concatenate([v, -v]).astype(np.float32)


def test_e2m1_matches_quantum_rounding():
    v = _e2m1_probe_values()
    got = np.array([oracle.e2m1_encode(x) for x in v], np.uint8)
    want = npref.e2m1_rne_quantum(v)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_grid_roundtrip_and_sign_of_zero():
    for code in range(16):
        val = npref.E2M1_LUT[code]
        assert oracle.e2m1_value(code) == val
        if code != 8:  # -0 encodes to 0x8 as well, checked below
            assert oracle.e2m1_encode(val) == code
    assert oracle.e2m1_encode(-0.0) == 0x8
    assert oracle.e2m1_encode(-0.2) == 0x8
    assert oracle.e2m1_encode(0.25) == 0x0      # tie 0 / 0.5 -> even code 0
    assert oracle.e2m1_encode(5.0) == 0x6       # tie 4 / 6 -> 4
    assert oracle.e2m1_encode(-100.0) == 0xF    # saturates to -6


def test_e4m3_values_match_torch():
    codes = np.arange(0x7F, dtype=np.uint8)
    want = npref.e4m3_values(codes)
    got = np.array([oracle.e4m3_value(c) for c in codes])
    np.testing.assert_array_equal(got, want)
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast():
    vals = npref.e4m3_values(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    pts = np.concatenate([vals, mids])
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                          np.nextafter(pts, np.float32(0))])
    b = _all_bf16_floats()
    rng = np.random.default_rng(2)
    s = np.concatenate([pts, b[(b >= 0) & (b < 464)],
                        rng.uniform(0, 464, 20000).astype(np.float32),
                        np.float32(2.0) ** rng.uniform(-30, -5, 5000).astype(np.float32)])
    s = s[(s >= 0) & (s < 464) & ~np.signbit(s)].astype(np.float32)
    got = np.array([oracle.e4m3_encode(x) for x in s], np.uint8)
    want = npref.e4m3_rne_torch(s)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (s[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_saturates_instead_of_nan():
    for s in [448.0, 449.0, 463.99, 464.0, 1e4, 3.4e38]:
        assert oracle.e4m3_encode(s) == 0x7E
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00   # tie 0 / 2^-9 -> even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie 2^-9 / 2^-8 -> even


def _read_kat():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x64_10_kat.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        words = [int(w, 16) for w in line.split()]
        rows.append((words[0:4], words[4:6], words[6:10]))
    return rows


def test_philox_known_answer():
    for ctr, key, want in _read_kat():
        got = oracle.philox4x64_10(ctr, key)
        assert [int(v) for v in got] == want


@pytest.mark.parametrize("seed", [0, 7, 12345])
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        ctr = [int(v) for v in rng.integers(1, 2**63, 4, dtype=np.uint64)]
        key = [int(v) for v in rng.integers(0, 2**63, 2, dtype=np.uint64)]
        # numpy's Philox increments the counter before each block
        bg = np.random.Philox(counter=[ctr[0] - 1] + ctr[1:], key=key)
        want = bg.random_raw(4)
        got = oracle.philox4x64_10(ctr, key)
        np.testing.assert_array_equal(got, want)
