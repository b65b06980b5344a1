"""Device-side preparation of the seeded layers (for benchmarks and tests).

Expert weights are drawn on the device by the counter-based generator
(libnvfp4synth) and quantized by the library's per-expert quantizer.
"""
from __future__ import annotations

import numpy as np

from . import binding, synth


def gpu_weights_rowmajor(layer_id: int, device="cuda", chunk: int = 16, n_experts: int | None = None):
    """NVFP4 weights of experts 0 .. n_experts - 1 (default: the layer's E;
    E + 1 adds a shared expert, generated like the others) in the row-major
    boundary layout, generated and quantized on the device."""
    import torch

    L = synth.LAYERS[layer_id]
    E = L.E if n_experts is None else n_experts
    (r13, c13), (r2, c2) = synth.weight_shapes(layer_id)
    k13 = synth.weight_key(layer_id, synth.WEIGHT_W13)
    k2 = synth.weight_key(layer_id, synth.WEIGHT_W2)
    out = []
    for key, (r, c) in ((k13, (r13, c13)), (k2, (r2, c2))):
        codes = torch.empty((E, r, c // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((E, r, c // 16), dtype=torch.uint8, device=device)
        g = torch.empty((E,), dtype=torch.float32, device=device)
        for e0 in range(0, E, chunk):
            n = min(chunk, E - e0)
            w = binding.synth_weights(*key, e0, n, (r, c), L.sigma, device=device)
            qc, qs, qg = binding.quantize_experts(w)
            codes[e0:e0 + n].copy_(qc)
            scales[e0:e0 + n].copy_(qs)
            g[e0:e0 + n].copy_(qg)
            del w, qc, qs, qg
        out += [codes, scales, g]
    torch.cuda.synchronize()
    return binding.NvFp4Weights(*out)


def gpu_weights(layer_id: int, device="cuda", chunk: int = 16, n_experts: int | None = None):
    """The same weights packed into unit records (binding.PackedWeights),
    generated, quantized and packed `chunk` experts at a time so that the
    row-major copy of the whole layer never exists at once."""
    import torch

    L = synth.LAYERS[layer_id]
    E = L.E if n_experts is None else n_experts
    (r13, c13), (r2, c2) = synth.weight_shapes(layer_id)
    k13 = synth.weight_key(layer_id, synth.WEIGHT_W13)
    k2 = synth.weight_key(layer_id, synth.WEIGHT_W2)
    packed = binding.PackedWeights.empty(E, L.H, L.I, device=device)
    for e0 in range(0, E, chunk):
        n = min(chunk, E - e0)
        parts = []
        for key, (r, c) in ((k13, (r13, c13)), (k2, (r2, c2))):
            w = binding.synth_weights(*key, e0, n, (r, c), L.sigma, device=device)
            parts += list(binding.quantize_experts(w))
            del w
        binding.pack_weights(binding.NvFp4Weights(*parts), out=packed.experts(e0, e0 + n))
        del parts
    torch.cuda.synchronize()
    return packed


def to_device_bf16(x_bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).to(device)


