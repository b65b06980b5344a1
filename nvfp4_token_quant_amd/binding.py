"""ctypes binding of the HIP library (include/nvfp4_moe.h).

Argument marshalling only: torch tensors supply device memory and the
current stream; every step of the layer runs in the library's kernels.  If
the library is missing this module raises on first use; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libnvfp4moe.so")
SYNTH_PATH = os.path.join(HERE, "libnvfp4synth.so")
HEADERS = [os.path.join(ROOT, "include", "nvfp4_moe.h"), os.path.join(ROOT, "include", "nvfp4_synth.h")]

MOE_DETERMINISTIC_FINALIZE = 0x1
MOE_STATIC_ACT_SCALES = 0x2
MOE_SHARED_EXPERT = 0x4
MOE_SHARED_AVERAGE = 0x8
MOE_W4A16 = 0x10

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_INVALID_ARG", 2: "NVFP4_ERR_TOO_MANY_TOKENS",
          3: "NVFP4_ERR_ALIAS", 4: "NVFP4_ERR_NO_WEIGHTS", 5: "NVFP4_ERR_METADATA_CHANGED",
          6: "NVFP4_ERR_HIP", 7: "NVFP4_ERR_OOM"}

BUF = dict(XQ_CODES=0, XQ_SCALES=1, XQ_GSCALE=2, TOPK_IDS=3, TOPK_W=4, COUNTS=5, OFFSETS=6,
           PERM=7, INV=8, ACT=9, A2_CODES=10, A2_SCALES=11, A2_GSCALE=12, A2_16=13)


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class MoeConfig(ctypes.Structure):
    _fields_ = [("max_num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int64), ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("w13_codes", ctypes.c_void_p), ("w13_scales", ctypes.c_void_p),
                ("w13_gscale", ctypes.c_void_p), ("w2_codes", ctypes.c_void_p),
                ("w2_scales", ctypes.c_void_p), ("w2_gscale", ctypes.c_void_p)]


class MoePacked(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int64), ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("w13", ctypes.c_void_p), ("w13_gscale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_gscale", ctypes.c_void_p)]


_lib = None
_synth = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run __graft_entry__.build() or nvfp4_token_quant_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_last_error.restype = ctypes.c_char_p
        L.nvfp4_last_error.argtypes = []
        L.nvfp4_quantize_per_token.restype = ctypes.c_int
        L.nvfp4_quantize_per_token.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
        L.nvfp4_quantize_experts.restype = ctypes.c_int
        L.nvfp4_quantize_experts.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]
        L.moe_workspace_create.restype = ctypes.c_int
        L.moe_workspace_create.argtypes = [ctypes.POINTER(MoeConfig), _P, ctypes.POINTER(_P)]
        L.moe_packed_bytes.restype = ctypes.c_int
        L.moe_packed_bytes.argtypes = [_I64, _I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [ctypes.POINTER(MoeWeights), _P, _P, _P]
        L.moe_workspace_bind_weights.restype = ctypes.c_int
        L.moe_workspace_bind_weights.argtypes = [_P, ctypes.POINTER(MoePacked), _P]
        L.moe_nvfp4_forward.restype = ctypes.c_int
        L.moe_nvfp4_forward.argtypes = [_P, _P, _P, _I64, _P, _P]
        L.moe_nvfp4_forward_quantized.restype = ctypes.c_int
        L.moe_nvfp4_forward_quantized.argtypes = [_P, _P, _P, _P, _P, _I64, _P, _P]
        L.refresh_scales_inplace.restype = ctypes.c_int
        L.refresh_scales_inplace.argtypes = [_P, ctypes.POINTER(MoeWeights), _P]
        L.moe_workspace_destroy.restype = ctypes.c_int
        L.moe_workspace_destroy.argtypes = [_P]
        L.moe_token_ceiling.restype = ctypes.c_int
        L.moe_token_ceiling.argtypes = [_I64, _I64, _I64, _I64, ctypes.POINTER(_I64)]
        L.moe_workspace_set_act_scales.restype = ctypes.c_int
        L.moe_workspace_set_act_scales.argtypes = [_P, _P, _P]
        L.moe_nvfp4_forward_noalloc.restype = ctypes.c_int
        L.moe_nvfp4_forward_noalloc.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoePacked), _P, _P,
                                                _I64, _P, _P]
        L.moe_workspace_buffer.restype = ctypes.c_int
        L.moe_workspace_buffer.argtypes = [_P, ctypes.c_int32, ctypes.POINTER(_P), ctypes.POINTER(_I64)]
        _lib = L
    return _lib


def synth_lib():
    global _synth
    if _synth is None:
        if not os.path.exists(SYNTH_PATH):
            raise ImportError(f"HIP library not built: {SYNTH_PATH} is missing")
        S = ctypes.CDLL(SYNTH_PATH)
        S.nvfp4_synth_weights.restype = ctypes.c_int
        S.nvfp4_synth_weights.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _I64, _I64, _I64,
                                          ctypes.c_double, _P, _P]
        S.nvfp4_synth_scale.restype = ctypes.c_float
        S.nvfp4_synth_scale.argtypes = [ctypes.c_double]
        S.nvfp4_synth_last_error.restype = ctypes.c_char_p
        _synth = S
    return _synth


def declared_functions():
    """Function names declared in include/*.h (for export checks)."""
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


def _check(rc: int):
    if rc != 0:
        raise Nvfp4Error(rc, lib().nvfp4_last_error().decode())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# --- quantization --------------------------------------------------------------

def quantize_per_token(x: torch.Tensor, stream=None):
    """x bf16 [rows, cols] (row stride may exceed cols) -> (codes u8 [rows, cols/2],
    scales u8 [rows, cols/16] (E4M3 bits), gscale f32 [rows])."""
    _require(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // 16, 0)), dtype=torch.uint8, device=x.device)
    g = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(lib().nvfp4_quantize_per_token(_ptr(x), rows, cols, x.stride(0) if rows else cols,
                                          _ptr(codes), _ptr(scales), _ptr(g), _stream(stream)))
    return codes, scales, g


def quantize_per_token_into(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                            g: torch.Tensor, stream=None):
    """quantize_per_token into caller-owned outputs (no allocation)."""
    _require(x, torch.bfloat16, "x")
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    _check(lib().nvfp4_quantize_per_token(_ptr(x), rows, cols, x.stride(0) if rows else cols,
                                          _ptr(codes), _ptr(scales), _ptr(g), _stream(stream)))
    return codes, scales, g


def quantize_experts(w: torch.Tensor, stream=None):
    """w f32 [E, rows, cols] -> (codes [E, rows, cols/2], scales [E, rows, cols/16], g [E])."""
    _require(w, torch.float32, "w")
    E, rows, cols = w.shape
    w = w.contiguous()
    codes = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device=w.device)
    g = torch.empty((E,), dtype=torch.float32, device=w.device)
    scratch = torch.empty((E,), dtype=torch.float32, device=w.device)
    _check(lib().nvfp4_quantize_experts(_ptr(w), E, rows, cols, _ptr(codes), _ptr(scales), _ptr(g),
                                        _ptr(scratch), _stream(stream)))
    return codes, scales, g


def token_ceiling(max_prefill, piecewise_max, graph_max_bs, spec_draft_tokens) -> int:
    out = ctypes.c_int64(0)
    _check(lib().moe_token_ceiling(max_prefill, piecewise_max, graph_max_bs, spec_draft_tokens,
                                   ctypes.byref(out)))
    return out.value


# --- synthetic weights (input generation) --------------------------------------

def synth_weights(seed: int, tag: int, expert0: int, experts: int, shape, sigma: float,
                  device="cuda", out=None, stream=None):
    n = 1
    for d in shape:
        n *= d
    if out is None:
        out = torch.empty((experts, *shape), dtype=torch.float32, device=device)
    rc = synth_lib().nvfp4_synth_weights(seed, tag, expert0, experts, n, sigma, _ptr(out),
                                         _stream(stream))
    if rc != 0:
        raise RuntimeError(synth_lib().nvfp4_synth_last_error().decode())
    return out


# --- MoE layer -------------------------------------------------------------------

class NvFp4Weights:
    """NVFP4 expert weights in the row-major boundary layout (torch device
    tensors).  Codes may be None (a scales-only descriptor, for
    refresh_scales and scale-only packing)."""

    def __init__(self, w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale):
        self.w13_codes, self.w13_scales, self.w13_gscale = w13_codes, w13_scales, w13_gscale
        self.w2_codes, self.w2_scales, self.w2_gscale = w2_codes, w2_scales, w2_gscale

    @property
    def dims(self):
        E, two_i, h16 = self.w13_scales.shape
        return E, h16 * 16, two_i // 2

    def desc(self, with_codes=True) -> MoeWeights:
        E, H, I = self.dims
        has = with_codes and self.w13_codes is not None
        return MoeWeights(E, H, I,
                          self.w13_codes.data_ptr() if has else None,
                          self.w13_scales.data_ptr(), self.w13_gscale.data_ptr(),
                          self.w2_codes.data_ptr() if has else None,
                          self.w2_scales.data_ptr(), self.w2_gscale.data_ptr())


def packed_bytes(num_experts, hidden, inter):
    """(W13 bytes, W2 bytes) of the packed unit records of num_experts experts."""
    b13, b2 = _I64(), _I64()
    _check(lib().moe_packed_bytes(num_experts, hidden, inter, ctypes.byref(b13), ctypes.byref(b2)))
    return b13.value, b2.value


class PackedWeights:
    """Expert weights packed into the kernels' unit records, in caller-owned
    device tensors: w13 / w2 uint8 [E, bytes per expert], global scales
    float32 [E].  A layer bound to them borrows the records (keep them
    alive); experts are contiguous, so [a:b] slices select experts."""

    def __init__(self, hidden, inter, w13, w13_gscale, w2, w2_gscale):
        self.hidden, self.inter = hidden, inter
        self.w13, self.w13_gscale, self.w2, self.w2_gscale = w13, w13_gscale, w2, w2_gscale

    @classmethod
    def empty(cls, num_experts, hidden, inter, device="cuda"):
        b13, b2 = packed_bytes(1, hidden, inter)
        return cls(hidden, inter,
                   torch.empty((num_experts, b13), dtype=torch.uint8, device=device),
                   torch.empty((num_experts,), dtype=torch.float32, device=device),
                   torch.empty((num_experts, b2), dtype=torch.uint8, device=device),
                   torch.empty((num_experts,), dtype=torch.float32, device=device))

    @property
    def num_experts(self):
        return self.w13.shape[0]

    def experts(self, a, b):
        """The packed weights of experts a .. b - 1 (views, no copy)."""
        return PackedWeights(self.hidden, self.inter, self.w13[a:b], self.w13_gscale[a:b],
                             self.w2[a:b], self.w2_gscale[a:b])

    def clone(self):
        return PackedWeights(self.hidden, self.inter, self.w13.clone(), self.w13_gscale.clone(),
                             self.w2.clone(), self.w2_gscale.clone())

    def desc(self) -> MoePacked:
        for t in (self.w13, self.w2, self.w13_gscale, self.w2_gscale):
            if not t.is_contiguous():
                raise ValueError("packed weight tensors must be contiguous")
        return MoePacked(self.num_experts, self.hidden, self.inter, self.w13.data_ptr(),
                         self.w13_gscale.data_ptr(), self.w2.data_ptr(), self.w2_gscale.data_ptr())


def pack_weights(w: NvFp4Weights, out: PackedWeights = None, stream=None) -> PackedWeights:
    """Pack row-major NVFP4 weights (moe_pack_weights) into `out` (new
    tensors if None); without codes in `w` only the scale bytes are written.
    The global scales are copied into out as well."""
    E, H, I = w.dims
    if out is None:
        out = PackedWeights.empty(E, H, I, device=w.w13_scales.device)
    if out.num_experts != E or out.hidden != H or out.inter != I:
        raise ValueError("packed buffers of other dims")
    d = w.desc(with_codes=w.w13_codes is not None)
    _check(lib().moe_pack_weights(ctypes.byref(d), _ptr(out.w13), _ptr(out.w2), _stream(stream)))
    out.w13_gscale.copy_(w.w13_gscale)
    out.w2_gscale.copy_(w.w2_gscale)
    return out


class MoeLayer:
    """Workspace + bound weights.  forward(x, logits) -> bf16 [T, H]."""

    def __init__(self, max_num_tokens, hidden, inter, num_experts, top_k, deterministic=True,
                 stream=None, static_act_scales=False, shared_expert=None, w4a16=False):
        """shared_expert: None, "sum" or "average" (the weights then hold
        num_experts + 1 experts, the last one shared by every token).
        w4a16: bf16 activations (no activation quantization), NVFP4 weights."""
        if shared_expert not in (None, "sum", "average"):
            raise ValueError("shared_expert must be None, 'sum' or 'average'")
        flags = (MOE_DETERMINISTIC_FINALIZE if deterministic else 0) | \
            (MOE_STATIC_ACT_SCALES if static_act_scales else 0) | \
            (MOE_SHARED_EXPERT if shared_expert else 0) | \
            (MOE_SHARED_AVERAGE if shared_expert == "average" else 0) | \
            (MOE_W4A16 if w4a16 else 0)
        self.cfg = MoeConfig(max_num_tokens, hidden, inter, num_experts, top_k, flags)
        h = ctypes.c_void_p()
        _check(lib().moe_workspace_create(ctypes.byref(self.cfg), _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.weights = None

    def bind(self, weights, stream=None):
        """Bind PackedWeights (borrowed: the layer keeps a reference), or
        NvFp4Weights, which are packed into new tensors first."""
        if isinstance(weights, NvFp4Weights):
            weights = pack_weights(weights, stream=stream)
        d = weights.desc()
        _check(lib().moe_workspace_bind_weights(self.handle, ctypes.byref(d), _stream(stream)))
        self.weights = weights

    def refresh_scales(self, weights: NvFp4Weights, stream=None):
        """New block and global scales (codes not read) written in place
        into the bound packed records and the layer's global scales."""
        d = weights.desc(with_codes=False)
        _check(lib().refresh_scales_inplace(self.handle, ctypes.byref(d), _stream(stream)))

    def set_act_scales(self, scales, stream=None):
        """Static global scales (g_x, g_a): float32 tensor of 2 on the device,
        copied into the workspace (workspaces made with static_act_scales)."""
        _require(scales, torch.float32, "scales")
        if scales.numel() != 2 or not scales.is_contiguous():
            raise ValueError("scales must be a contiguous float32 tensor of 2 values (g_x, g_a)")
        _check(lib().moe_workspace_set_act_scales(self.handle, _ptr(scales), _stream(stream)))

    def forward_into(self, x, logits, out, T=None, stream=None):
        T = x.shape[0] if T is None else T
        _check(lib().moe_nvfp4_forward(self.handle, _ptr(x), _ptr(logits), T, _ptr(out),
                                       _stream(stream)))
        return out

    def forward(self, x, logits, stream=None):
        _require(x, torch.bfloat16, "x")
        _require(logits, torch.float32, "logits")
        x = x.contiguous()
        logits = logits.contiguous()
        out = torch.empty_like(x)
        return self.forward_into(x, logits, out, stream=stream)

    def forward_quantized_into(self, codes, scales, gscale, logits, out, T=None, stream=None):
        T = codes.shape[0] if T is None else T
        _check(lib().moe_nvfp4_forward_quantized(self.handle, _ptr(codes), _ptr(scales), _ptr(gscale),
                                                 _ptr(logits), T, _ptr(out), _stream(stream)))
        return out

    def forward_quantized(self, codes, scales, gscale, logits, stream=None):
        """The forward for activations already quantized per token: codes
        uint8 [T, H/2], scales uint8 [T, H/16] (E4M3 bits), gscale float32
        [T] (as quantize_per_token returns them); bf16 [T, H] out."""
        _require(codes, torch.uint8, "codes")
        _require(scales, torch.uint8, "scales")
        _require(gscale, torch.float32, "gscale")
        _require(logits, torch.float32, "logits")
        T = codes.shape[0]
        H = codes.shape[1] * 2
        if tuple(scales.shape) != (T, H // 16) or tuple(gscale.shape) != (T,):
            raise ValueError("scales must be [T, H/16] and gscale [T] for codes [T, H/2]")
        codes, scales, gscale, logits = (t.contiguous() for t in (codes, scales, gscale, logits))
        out = torch.empty((T, H), dtype=torch.bfloat16, device=codes.device)
        return self.forward_quantized_into(codes, scales, gscale, logits, out, stream=stream)

    def buffer(self, name: str):
        """(device pointer, bytes) of an intermediate buffer."""
        p = ctypes.c_void_p()
        n = ctypes.c_int64()
        _check(lib().moe_workspace_buffer(self.handle, BUF[name], ctypes.byref(p), ctypes.byref(n)))
        return p.value, n.value

    def read_buffer(self, name: str, dtype: torch.dtype, shape):
        """Copy the leading part of an intermediate buffer into a new tensor."""
        ptr, nbytes = self.buffer(name)
        out = torch.empty(shape, dtype=dtype, device="cuda")
        want = out.numel() * out.element_size()
        if want > nbytes:
            raise ValueError(f"{name}: {want} bytes requested, buffer holds {nbytes}")
        torch.cuda.synchronize()
        _hip_memcpy_d2d(out.data_ptr(), ptr, want)
        return out

    def close(self):
        if self.handle:
            lib().moe_workspace_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward_noalloc(cfg: MoeConfig, weights: PackedWeights, x, logits, out, T=None, stream=None):
    """moe_nvfp4_forward_noalloc: the forward with no workspace and no
    allocation (intermediates in the library's fixed device array)."""
    T = x.shape[0] if T is None else T
    d = weights.desc()
    _check(lib().moe_nvfp4_forward_noalloc(ctypes.byref(cfg), ctypes.byref(d), _ptr(x), _ptr(logits), T,
                                           _ptr(out), _stream(stream)))
    return out


_hip = None


def _hip_memcpy_d2d(dst, src, nbytes):
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [_P, _P, ctypes.c_size_t, ctypes.c_int]
    rc = _hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 3)  # device to device
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
