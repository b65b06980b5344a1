"""CPU oracle of the NVFP4 fused-MoE layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never imports it.  The arithmetic lives in
``nvfp4_oracle.cpp``; this module only marshals numpy arrays.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(exhaustive encoder checks, library cross-checks, closed forms, the lossless
special case and the brute-force dense layer); see each test's docstring.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _declare(L):
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_e2m1_encode.argtypes = [ctypes.c_float]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_global_scale.restype = ctypes.c_float
    L.orc_global_scale.argtypes = [_P, _I64]
    for name in ("orc_quantize_rows", "orc_quantize_rows_bf16"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.orc_quantize_rows_given_g.restype = None
    L.orc_quantize_rows_given_g.argtypes = [_P, _I64, _I64, _P, _P, _P]
    L.orc_quantize_groups.restype = None
    L.orc_quantize_groups.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
    L.orc_dequantize.restype = None
    L.orc_dequantize.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
    L.orc_router.restype = None
    L.orc_router.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.orc_permute.restype = None
    L.orc_permute.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
    L.orc_moe_layer.restype = ctypes.c_int
    _F = ctypes.c_float
    L.orc_moe_layer.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64,
                                _P, _P, _P, _P, _P, _P, _F, _F, ctypes.c_int, _P, _P, _P, _P, _P, _P]
    L.orc_moe_layer_xq.restype = ctypes.c_int
    L.orc_moe_layer_xq.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64,
                                   _P, _P, _P, _P, _P, _P, _F, _P]
    L.orc_moe_layer_dense.restype = None
    L.orc_moe_layer_dense.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                      _P, _P, _P, _P, _P, _P, _F, _F, ctypes.c_int, _P]
    L.orc_f32_to_bf16.restype = None
    L.orc_f32_to_bf16.argtypes = [_P, _I64, _P]
    L.orc_philox4x64_10.restype = None
    L.orc_philox4x64_10.argtypes = [_P, _P, _P]
    L.orc_synth_scale.restype = ctypes.c_float
    L.orc_synth_scale.argtypes = [ctypes.c_double]
    L.orc_synth_weights.restype = None
    L.orc_synth_weights.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _I64, _I64,
                                    ctypes.c_double, _P]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_num_threads.argtypes = []


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- encoders ---------------------------------------------------------------

def e2m1_encode(v: float) -> int:
    return int(lib().orc_e2m1_encode(float(v)))


def e2m1_value(code: int) -> float:
    return float(lib().orc_e2m1_value(int(code)))


def e4m3_encode(s: float) -> int:
    return int(lib().orc_e4m3_encode(float(s)))


def e4m3_value(b: int) -> float:
    return float(lib().orc_e4m3_value(int(b)))


# --- quantization -----------------------------------------------------------

def global_scale(x) -> np.float32:
    x = _c(x, np.float32).ravel()
    return np.float32(lib().orc_global_scale(_p(x), x.size))


def quantize_rows(x):
    """Per-row NVFP4: x float32 [rows, K] or bf16 bits (uint16) [rows, K].

    Returns (codes u8 [rows, K/2], scales u8 [rows, K/16], g f32 [rows]).
    """
    x = np.asarray(x)
    rows, K = x.shape
    codes = np.empty((rows, K // 2), np.uint8)
    S = np.empty((rows, K // 16), np.uint8)
    g = np.empty(rows, np.float32)
    if x.dtype == np.uint16:
        x = _c(x, np.uint16)
        lib().orc_quantize_rows_bf16(_p(x), rows, K, _p(codes), _p(S), _p(g))
    else:
        x = _c(x, np.float32)
        lib().orc_quantize_rows(_p(x), rows, K, _p(codes), _p(S), _p(g))
    return codes, S, g


def quantize_rows_given_g(x, g):
    x = _c(x, np.float32)
    rows, K = x.shape
    g = _c(np.broadcast_to(np.asarray(g, np.float32), (rows,)), np.float32)
    codes = np.empty((rows, K // 2), np.uint8)
    S = np.empty((rows, K // 16), np.uint8)
    lib().orc_quantize_rows_given_g(_p(x), rows, K, _p(g), _p(codes), _p(S))
    return codes, S


def quantize_groups(x):
    """Per-group (expert) NVFP4 of float32 [G, rows, K] -> codes, scales, g [G]."""
    x = _c(x, np.float32)
    G, rows, K = x.shape
    codes = np.empty((G, rows, K // 2), np.uint8)
    S = np.empty((G, rows, K // 16), np.uint8)
    g = np.empty(G, np.float32)
    lib().orc_quantize_groups(_p(x), G, rows, K, _p(codes), _p(S), _p(g))
    return codes, S, g


def dequantize(codes, S, g, g_stride_rows=1):
    codes = _c(codes, np.uint8)
    S = _c(S, np.uint8)
    g = _c(g, np.float32).ravel()
    K = codes.shape[-1] * 2
    rows = codes.size // (K // 2)
    out = np.empty(rows * K, np.float64)
    lib().orc_dequantize(_p(codes), _p(S), _p(g), rows, K, g_stride_rows, _p(out))
    return out.reshape(codes.shape[:-1] + (K,))


# --- router / permutation ----------------------------------------------------

def router(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_router(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    lib().orc_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


# --- layer --------------------------------------------------------------------

class QuantWeights:
    """Compact NVFP4 weights for a subset of experts (oracle side)."""

    def __init__(self, experts, w13c, w13s, w13g, w2c, w2s, w2g):
        self.experts = _c(experts, np.int32)
        self.w13c, self.w13s, self.w13g = _c(w13c, np.uint8), _c(w13s, np.uint8), _c(w13g, np.float32)
        self.w2c, self.w2s, self.w2g = _c(w2c, np.uint8), _c(w2s, np.uint8), _c(w2g, np.float32)


def moe_layer(x_bf16, ids, w, tokens, H, I, qw: QuantWeights, debug=False, static_scales=None,
              a16=False):
    """Layer output (float64 [n_tok, H]) for the listed tokens.

    x_bf16: uint16 [T, H]; ids int32 [T, k]; w float64 [T, k] (from router()).
    static_scales: None (per-row global scales) or (g_x, g_a), the static
    global scales of x and of the GEMM2 input.
    a16: W4A16 — x itself (bf16) and the SwiGLU output rounded to bf16
    (round to nearest even) are the GEMM inputs; the activations are not
    quantized (the debug c2 / S2 / g2 are then not written).
    With debug=True also returns a dict of per-slot intermediates.
    """
    gx, ga = (0.0, 0.0) if static_scales is None else static_scales
    x_bf16 = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    tokens = _c(tokens, np.int64)
    k = ids.shape[1]
    n = tokens.size
    out = np.empty((n, H), np.float64)
    dbg = None
    if debug:
        dbg = dict(y=np.empty((n, k, H), np.float64), act=np.empty((n, k, I), np.float32),
                   c2=np.empty((n, k, I // 2), np.uint8), S2=np.empty((n, k, I // 16), np.uint8),
                   g2=np.empty((n, k), np.float32))
    rc = lib().orc_moe_layer(
        _p(x_bf16), _p(ids), _p(w), _p(tokens), n, H, I, k, _p(qw.experts), qw.experts.size,
        _p(qw.w13c), _p(qw.w13s), _p(qw.w13g), _p(qw.w2c), _p(qw.w2s), _p(qw.w2g),
        float(np.float32(gx)), float(np.float32(ga)), int(bool(a16)), _p(out),
        _p(dbg["y"]) if debug else None, _p(dbg["act"]) if debug else None,
        _p(dbg["c2"]) if debug else None, _p(dbg["S2"]) if debug else None,
        _p(dbg["g2"]) if debug else None)
    if rc != 0:
        raise ValueError("a routed expert is missing from the compact weights")
    return (out, dbg) if debug else out


def moe_layer_quantized(xq_codes, xq_scales, xq_g, ids, w, tokens, H, I, qw: QuantWeights,
                        static_ga=None):
    """Layer output (float64 [n_tok, H]) for activations handed over already
    quantized: xq_codes u8 [T, H/2], xq_scales u8 [T, H/16] (E4M3 bits),
    xq_g f32 [T] (encode-direction global scales, value = code x scale / g).

    [P1] "Implementation breakdown" item 2: the runner receives the FP4
    codes, the block scales and the per-token scale.  The layer's first step
    (Q of x) is replaced by these rows; the rest is moe_layer's.
    static_ga: None (per-row re-quantization scales) or the static global
    scale of the GEMM2 input.
    """
    xq_codes = _c(xq_codes, np.uint8)
    xq_scales = _c(xq_scales, np.uint8)
    xq_g = _c(xq_g, np.float32).ravel()
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    tokens = _c(tokens, np.int64)
    k = ids.shape[1]
    n = tokens.size
    out = np.empty((n, H), np.float64)
    ga = 0.0 if static_ga is None else float(np.float32(static_ga))
    rc = lib().orc_moe_layer_xq(
        _p(xq_codes), _p(xq_scales), _p(xq_g), _p(ids), _p(w), _p(tokens), n, H, I, k,
        _p(qw.experts), qw.experts.size, _p(qw.w13c), _p(qw.w13s), _p(qw.w13g), _p(qw.w2c),
        _p(qw.w2s), _p(qw.w2g), ga, _p(out))
    if rc != 0:
        raise ValueError("a routed expert is missing from the compact weights")
    return out


def moe_layer_shared(x_bf16, ids, w, tokens, H, I, qw: QuantWeights, shared: QuantWeights,
                     strategy="sum", static_scales=None, a16=False):
    """Routed output plus a shared expert's output for the listed tokens.

    [P3] Command-A-Plus multi-stream page, Cohere2MoeSparseMoeBlock.forward:
    the shared expert runs on the same input as the routed experts, the two
    outputs are added, and the 'average' combination strategy halves the sum.
    The shared expert is an NVFP4 expert of the routed experts' shape applied
    to every token with weight 1, its input quantized per token exactly as
    the routed experts' (the same Q of x, the same re-quantization of its
    act): it is the routed layer with one slot per token, all routed to it.
    shared: QuantWeights holding that one expert (any expert id).
    strategy: "sum" or "average".
    """
    if strategy not in ("sum", "average"):
        raise ValueError("strategy must be 'sum' or 'average'")
    if shared.experts.size != 1:
        raise ValueError("shared holds exactly one expert")
    x_bf16 = _c(x_bf16, np.uint16)
    routed = moe_layer(x_bf16, ids, w, tokens, H, I, qw, static_scales=static_scales, a16=a16)
    T = x_bf16.shape[0]
    ids_s = np.full((T, 1), shared.experts[0], np.int32)
    w_s = np.ones((T, 1), np.float64)
    out = routed + moe_layer(x_bf16, ids_s, w_s, tokens, H, I, shared, static_scales=static_scales,
                             a16=a16)
    return out / 2 if strategy == "average" else out


def moe_layer_dense(x_bf16, ids, w, H, I, E, w13c, w13s, w13g, w2c, w2s, w2g, static_scales=None,
                    a16=False):
    x_bf16 = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, k = ids.shape
    args = [_c(a, np.uint8) if a.dtype == np.uint8 else _c(a, np.float32)
            for a in (w13c, w13s, w13g, w2c, w2s, w2g)]
    out = np.empty((T, H), np.float64)
    gx, ga = (0.0, 0.0) if static_scales is None else static_scales
    lib().orc_moe_layer_dense(_p(x_bf16), _p(ids), _p(w), T, H, I, E, k,
                              *[_p(a) for a in args], float(np.float32(gx)), float(np.float32(ga)),
                              int(bool(a16)), _p(out))
    return out


def f32_to_bf16(x):
    """binary32 -> bfloat16 bits (uint16), round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16(_p(x), x.size, _p(out))
    return out


# --- synthetic weights (input generation) -----------------------------------

def philox4x64_10(ctr, key):
    c = np.asarray(ctr, np.uint64)
    kk = np.asarray(key, np.uint64)
    o = np.empty(4, np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(kk), _p(o))
    return o


def synth_scale(sigma):
    return np.float32(lib().orc_synth_scale(float(sigma)))


def synth_weights(seed, tag, expert, shape, sigma):
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    lib().orc_synth_weights(seed, tag, expert, n, float(sigma), _p(out))
    return out.reshape(shape)


def num_threads():
    return int(lib().orc_num_threads())
