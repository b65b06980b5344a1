"""Seeded synthetic inputs for the NVFP4 MoE layer.

This module holds input generation only (no step of the method): the same
arrays feed the HIP path and the CPU oracle.  Expert weights are too large to
draw on the host for the biggest layer, so they come from a counter-based
generator (Philox4x64-10, Salmon et al., SC'11) that each side implements
itself from the published definition; this module fixes only its key and tag
scheme (``weight_key``) and the spread ``sigma``.

Workloads (the pages measure end-to-end serving with trained checkpoints on
GSM8K, which are not available; these seeded layers stand in for them):

==  =====  =====  ===  ==  ====  ==============================================
id  T      H      E    k   I     activations / routing
==  =====  =====  ===  ==  ====  ==============================================
1   16     256    8    2   512   x ~ N(0,1); logits ~ N(0,1)
2   64     2048   128  8   768   x ~ N(0,1), 20 seeded channels x20; logits ~ N(0,1.5^2)
3   4096   2048   128  8   768   as 2; logits = log p_zipf(1.1) + Gumbel
4   16384  7168   -    -   -     quantize only: x ~ Student-t(3), every 97th row 0,
                                 4 seeded nonzero rows x1e3
5   1/7/2048 7168 256  8   2048  x ~ N(0,1); logits = log p_zipf(1.2) + Gumbel,
                                 8 seeded experts pinned to logit -30 (never routed);
                                 workspace ceiling 8192 tokens
==  =====  =====  ===  ==  ====  ==============================================

Weights: sigma 0.02 (layers 1-3), 0.01 (layer 5); quantized to NVFP4 with a
per-expert global scale by whichever side consumes them.

RNG: numpy ``Generator(PCG64(SeedSequence([seed, layer_id, tensor_id])))``,
seed 0, fixed draw order; bf16 values are round-to-nearest-even from float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SEED = 0
TENSOR_X = 0
TENSOR_LOGITS = 1
WEIGHT_W13 = 1
WEIGHT_W2 = 2


@dataclass(frozen=True)
class Layer:
    id: int
    name: str
    T: int
    H: int
    E: int = 0
    k: int = 0
    I: int = 0
    sigma: float = 0.0
    max_tokens: int = 0


LAYERS = {
    1: Layer(1, "tiny", 16, 256, 8, 2, 512, 0.02, 16),
    2: Layer(2, "decode", 64, 2048, 128, 8, 768, 0.02, 64),
    3: Layer(3, "prefill", 4096, 2048, 128, 8, 768, 0.02, 4096),
    4: Layer(4, "quantize", 16384, 7168),
    5: Layer(5, "large", 2048, 7168, 256, 8, 2048, 0.01, 8192),
    # Shapes at the edges of what the library accepts (tests only): one
    # expert and one K step in both GEMMs; more experts than the one-launch
    # prologues take, the largest top-k, an odd number of K steps and a
    # GEMM2 unit count not divisible by four; the tiled GEMMs with partial
    # column bands; the largest expert count; 256 experts on small shapes
    # (both routers of the one-block prologue on the most keys per lane);
    # the largest top-k on the 64-token routing blocks (1024 (t, j) entries
    # per block) with the tiled GEMMs.
    6: Layer(6, "edge-single", 9, 128, 1, 1, 128, 0.02, 16),
    7: Layer(7, "edge-wide", 33, 384, 300, 16, 384, 0.02, 64),
    8: Layer(8, "edge-tiled", 700, 640, 6, 3, 256, 0.02, 1024),
    9: Layer(9, "edge-experts", 3, 256, 1024, 16, 128, 0.02, 8),
    10: Layer(10, "edge-router", 8, 128, 256, 8, 128, 0.02, 64),
    11: Layer(11, "edge-topk16", 300, 256, 64, 16, 128, 0.02, 512),
}


def _rng(layer_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, layer_id, tensor_id])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations(layer_id: int, T: int | None = None) -> np.ndarray:
    """x as bf16 bits, uint16 [T, H]."""
    L = LAYERS[layer_id]
    T = L.T if T is None else T
    rng = _rng(layer_id, TENSOR_X)
    if layer_id == 4:
        x = rng.standard_t(3, size=(T, L.H)).astype(np.float32)
        x[np.arange(T) % 97 == 0] = 0.0
        candidates = np.flatnonzero(np.arange(T) % 97 != 0)
        big = rng.choice(candidates, size=min(4, candidates.size), replace=False)
        x[big] *= np.float32(1e3)
    elif layer_id in (2, 3):
        channels = rng.choice(L.H, size=L.H // 100, replace=False)
        x = rng.standard_normal((T, L.H), dtype=np.float32)
        x[:, channels] *= np.float32(20.0)
    else:
        x = rng.standard_normal((T, L.H), dtype=np.float32)
    return bf16_bits(x)


def outlier_channels(layer_id: int) -> np.ndarray:
    """The channels scaled x20 in layers 2 and 3 (same draw as activations())."""
    L = LAYERS[layer_id]
    return np.sort(_rng(layer_id, TENSOR_X).choice(L.H, size=L.H // 100, replace=False))


def zipf_probs(E: int, s: float) -> np.ndarray:
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def router_logits(layer_id: int, T: int | None = None) -> np.ndarray:
    """Router logits, float32 [T, E]."""
    L = LAYERS[layer_id]
    T = L.T if T is None else T
    rng = _rng(layer_id, TENSOR_LOGITS)
    if layer_id == 1:
        return rng.standard_normal((T, L.E), dtype=np.float32)
    if layer_id == 2:
        return (rng.standard_normal((T, L.E), dtype=np.float32) * np.float32(1.5)).astype(np.float32)
    s = 1.1 if layer_id == 3 else 1.2
    rank_to_expert = rng.permutation(L.E)
    logp = np.empty(L.E, np.float64)
    logp[rank_to_expert] = np.log(zipf_probs(L.E, s))
    gumbel = rng.gumbel(size=(T, L.E))
    logits = (logp[None, :] + gumbel).astype(np.float32)
    if layer_id == 5:
        logits[:, cold_experts(5)] = np.float32(-30.0)
    return logits


def cold_experts(layer_id: int) -> np.ndarray:
    """Experts of layer 5 pinned to logit -30 (they receive no tokens)."""
    assert layer_id == 5
    rng = _rng(layer_id, 2)
    return np.sort(rng.choice(LAYERS[5].E, size=8, replace=False))


def weight_key(layer_id: int, which: int) -> tuple[int, int]:
    """Philox key (seed, tag) of a layer's w13 (which=1) or w2 (which=2)."""
    return SEED, layer_id * 16 + which


def weight_shapes(layer_id: int):
    """Per-expert shapes: w13 [2I, H], w2 [H, I]."""
    L = LAYERS[layer_id]
    return (2 * L.I, L.H), (L.H, L.I)


def synth_scale_reference(sigma: float) -> float:
    """sigma / sqrt(4 (2^32 - 1) / 12): the Irwin-Hall(4) scale, for docs/tests."""
    return sigma / math.sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0)
