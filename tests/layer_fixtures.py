"""Shared set-up of the seeded layers for the tests.

Inputs (x, logits) come from nvfp4_token_quant_amd.synth; expert weights come
from the counter-based generator, implemented once on each side: the oracle's
C code for the CPU reference and the device generator for the HIP path.  Each
side quantizes its own copy (the oracle's Q on the CPU, the library's
nvfp4_quantize_experts on the GPU); tests compare the two bit for bit.
"""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
from nvfp4_token_quant_amd import synth
from nvfp4_token_quant_amd.workloads import gpu_weights, to_device_bf16  # noqa: F401

TOL_REL = 5e-3        # ||gpu - ref|| / ||ref||
TOL_MAX_RMS = 3e-2    # max |gpu - ref| / rms(ref)


def bf16_half_ulp(v):
    """Half a bf16 unit in the last place at |v| (bf16 keeps 8 significant
    bits: for |v| in [2^e, 2^(e+1)) the spacing is 2^(e-7)); the smallest
    normal spacing below 2^-126."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 8).astype(np.int64))


def check_layer_tolerance(got, ref):
    """The layer tolerance: ||gpu - ref|| / ||ref|| <= 5e-3, and every
    element within 3e-2 * rms(ref) of the binary64 reference beyond the
    rounding of the bf16 output itself.  The output is bf16 (the layer
    returns the model's dtype), so even a perfect layer differs from the
    unrounded reference by up to half a bf16 ulp, 2^-9 of |out|: more than
    3e-2 * rms wherever |out| > 7.7 rms, as happens on the prefill-shaped
    layer's largest outputs (9 - 12 rms).  The max bound is therefore applied
    to |gpu - ref| minus half a bf16 ulp at max(|gpu|, |ref|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite layer output"
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rms = np.sqrt((ref ** 2).mean())
    d = np.abs(got - ref)
    raw = d.max() / rms
    mx = (d - bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref)))).max() / rms
    print(f"layer tolerance: rel {rel:.3e}, max/rms beyond rounding {mx:.3e} (raw {raw:.3e}), "
          f"{got.size} outputs", file=sys.stderr, flush=True)
    assert rel <= TOL_REL and mx <= TOL_MAX_RMS, f"rel {rel:.3e}, max/rms beyond rounding {mx:.3e} (raw {raw:.3e})"
    return rel, mx


_prepared = set()


@functools.lru_cache(maxsize=None)
def oracle_expert(layer_id: int, e: int):
    """(w13 codes, scales, g, w2 codes, scales, g) of one expert, oracle side."""
    L = synth.LAYERS[layer_id]
    (r13, c13), (r2, c2) = synth.weight_shapes(layer_id)
    w13 = oracle.synth_weights(*synth.weight_key(layer_id, synth.WEIGHT_W13), e, (r13, c13), L.sigma)
    q13 = oracle.quantize_groups(w13[None])
    del w13
    w2 = oracle.synth_weights(*synth.weight_key(layer_id, synth.WEIGHT_W2), e, (r2, c2), L.sigma)
    q2 = oracle.quantize_groups(w2[None])
    return tuple(a[0] for a in q13) + tuple(a[0] for a in q2)


def oracle_weights(layer_id: int, experts) -> oracle.QuantWeights:
    experts = sorted(set(int(e) for e in experts))
    new = [e for e in experts if (layer_id, e) not in _prepared]
    if len(new) > 16:
        print(f"oracle: preparing {len(new)} experts of layer {layer_id}", file=sys.stderr, flush=True)
    parts = []
    for i, e in enumerate(experts):
        parts.append(oracle_expert(layer_id, e))
        _prepared.add((layer_id, e))
        if len(new) > 16 and (i + 1) % 64 == 0:
            print(f"oracle: {i + 1} of {len(experts)} experts ready", file=sys.stderr, flush=True)
    stack = [np.stack([p[i] for p in parts]) for i in range(6)]
    return oracle.QuantWeights(np.array(experts, np.int32), *stack)


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64)


# Row-group counts of the tiled GEMM kernel's tile variants (a tile of r rows
# computes the smallest variant holding ceil(r / 16) groups of 16 rows).
TILE_VARIANTS = (1, 2, 3, 4, 6, 8)
TILE_ROWS = 128


def tile_variant(rows: int) -> int:
    groups = (rows + 15) // 16
    return next(v for v in TILE_VARIANTS if v >= groups)


def covering_tokens(ids, E, mt=TILE_ROWS):
    """Tokens whose expanded rows include every active expert's first and
    last row in the stable expandInputRows order (so the first and the last
    tile of every expert), plus the tile variants present in the whole tile
    list and those the chosen rows sit in.  Middle tiles are full (variant
    8), as is the first tile of any expert with at least mt rows."""
    k = ids.shape[1]
    counts, offsets, perm, _ = oracle.permute(ids, E)
    rows, present, covered = [], set(), set()
    for e in np.flatnonzero(counts):
        c, o = int(counts[e]), int(offsets[e])
        rows += [o, o + c - 1]
        nt = (c + mt - 1) // mt
        for i in range(nt):
            present.add(tile_variant(min(mt, c - i * mt)))
        covered.add(tile_variant(min(mt, c)))
        covered.add(tile_variant(c - (nt - 1) * mt))
    toks = np.unique(perm[np.array(rows, np.int64)] // k)
    return toks, present, covered


def check_act_rows(act_gpu, inv, dbg_act, toks, k, rel=1e-4):
    """GPU SwiGLU output of the listed tokens' expanded rows against the
    oracle's (fp32 MFMA accumulation against binary64 dot products): every
    element within rel x the largest |act| of its row."""
    for ti, t in enumerate(toks):
        for j in range(k):
            got = act_gpu[inv[t * k + j]].astype(np.float64)
            ref = dbg_act[ti, j].astype(np.float64)
            scale = np.abs(ref).max()
            assert np.abs(got - ref).max() <= rel * scale, f"token {t} slot {j}"
