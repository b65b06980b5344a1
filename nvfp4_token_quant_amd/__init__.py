"""MI355X-native NVFP4 fused-MoE layer with online per-token activation quantization.

The compute lives in a HIP library (``libnvfp4moe.so``, gfx950) behind a
C-ABI; ``nvfp4_token_quant_amd.binding`` marshals torch tensors into it.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
__all__ = ["binding", "synth"]
