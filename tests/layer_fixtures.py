"""Shared set-up of the seeded layers for the tests.

Inputs (x, logits) come from nvfp4_token_quant_amd.synth; expert weights come
from the counter-based generator, implemented once on each side: the oracle's
C code for the CPU reference and the device generator for the HIP path.  Each
side quantizes its own copy (the oracle's Q on the CPU, the library's
nvfp4_quantize_experts on the GPU); tests compare the two bit for bit.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
from nvfp4_token_quant_amd import synth
from nvfp4_token_quant_amd.workloads import gpu_weights, to_device_bf16  # noqa: F401

TOL_REL = 5e-3        # ||gpu - ref|| / ||ref||
TOL_MAX_RMS = 3e-2    # max |gpu - ref| / rms(ref)


def check_layer_tolerance(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite layer output"
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max() / np.sqrt((ref ** 2).mean())
    assert rel <= TOL_REL and mx <= TOL_MAX_RMS, f"rel {rel:.3e}, max/rms {mx:.3e}"
    return rel, mx


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
    parts = [oracle_expert(layer_id, e) for e in experts]
    stack = [np.stack([p[i] for p in parts]) for i in range(6)]
    return oracle.QuantWeights(np.array(experts, np.int32), *stack)


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    return t.float().cpu().numpy().astype(np.float64)
