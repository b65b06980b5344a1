"""Independent numpy formulations used by the oracle's pins (tests only).

Each helper restates a format or a step a second way (a different algorithm
or a library routine), so that a mistake in the oracle's own code shows up as
a mismatch instead of being copied into the check.
"""
import numpy as np
import torch

# OCP MX FP4 E2M1 values by 4-bit code (sign in bit 3).
E2M1_LUT = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6],
                    np.float64)


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """E4M3 byte -> value through torch's float8_e4m3fn dtype (library)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def e4m3_rne_torch(s: np.ndarray) -> np.ndarray:
    """binary32 -> E4M3 byte via torch's cast (library; valid below 464)."""
    t = torch.from_numpy(np.ascontiguousarray(s, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def e2m1_rne_quantum(v: np.ndarray) -> np.ndarray:
    """E2M1 encode as a binary float format (2 exponent bits, bias 1, 1
    mantissa bit): round |v| to a multiple of its binade's quantum with
    ties-to-even (np.rint), saturate at 6, keep the sign bit."""
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    expo = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.where(a >= 1.0, 2.0 ** (expo - 1), 0.5)
    r = np.minimum(np.rint(a / q) * q, 6.0)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    idx = np.searchsorted(mags, r)
    assert np.all(mags[idx] == r)
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """Packed bytes [..., K/2] -> 4-bit codes [..., K], low nibble first."""
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def dequant(codes, S, g, g_per_row=True):
    """NVFP4 -> float64 via lookup tables: value(c) * value(S) / g."""
    c = unpack_codes(codes)
    vals = E2M1_LUT[c]
    d = np.repeat(e4m3_values(S), 16, axis=-1)
    g = np.asarray(g, np.float64)
    if g_per_row:
        g = g[..., None]
    return vals * d / g
