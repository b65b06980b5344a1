"""Host-side checks of the C-ABI library (no GPU needed).

The library must load and export every function its headers declare; the
argument checks that run before any device work must reject bad input with
the documented status; the token-ceiling helper reproduces the three cases
printed on the sglang PR #26696 report ("Source snippets",
TestCutedslMoeMaxNumTokens): 16384, 4096 and 512.
"""
import ctypes

import pytest

from nvfp4_token_quant_amd import binding


def test_library_exports_every_declared_symbol():
    names = binding.declared_functions()
    assert "moe_nvfp4_forward" in names and "nvfp4_quantize_per_token" in names
    L = binding.lib()
    S = binding.synth_lib()
    for n in names:
        assert hasattr(L, n) or hasattr(S, n), n


def test_token_ceiling_cases_from_the_pages():
    # default: max_prefill 16384 dominates piecewise 2048 and graph bs 512
    assert binding.token_ceiling(16384, 2048, 512, 0) == 16384
    # speculative decoding with 8 draft tokens: 512 * 8 = 4096
    assert binding.token_ceiling(512, 512, 512, 8) == 4096
    # piecewise graphs disabled, graph bs 64: prefill 512 dominates
    assert binding.token_ceiling(512, 0, 64, 0) == 512
    with pytest.raises(binding.Nvfp4Error) as ei:
        binding.token_ceiling(-1, 0, 0, 0)
    assert ei.value.status == "NVFP4_ERR_INVALID_ARG"


def _qpt(rows, cols, ld, x=16, c=16, s=16, g=16):
    return binding.lib().nvfp4_quantize_per_token(ctypes.c_void_p(x), rows, cols, ld,
                                                  ctypes.c_void_p(c), ctypes.c_void_p(s),
                                                  ctypes.c_void_p(g), None)


def test_quantize_argument_checks():
    L = binding.lib()
    assert _qpt(4, 15, 16) == 1                     # cols not a multiple of 16
    assert _qpt(4, 32, 24) == 1                     # ld_x < cols
    assert _qpt(4, 32, 36) == 1                     # ld_x not a multiple of 8
    assert _qpt(-1, 32, 32) == 1
    assert _qpt(0, 32, 32) == 0                     # empty input: no-op
    assert _qpt(4, 32, 32, x=0) == 1                # NULL
    assert _qpt(4, 32, 32, x=8) == 1                # misaligned x
    assert _qpt(4, 32, 32, x=4096, c=4096 + 64) == 3  # codes inside x
    assert b"overlap" in L.nvfp4_last_error()


def test_workspace_config_checks():
    L = binding.lib()
    h = ctypes.c_void_p()
    for cfg in [(0, 2048, 768, 128, 8, 1), (64, 2000, 768, 128, 8, 1), (64, 2048, 700, 128, 8, 1),
                (64, 2048, 768, 0, 8, 1), (64, 2048, 768, 4, 8, 1), (64, 2048, 768, 128, 17, 1),
                (64, 2048, 768, 2000, 8, 1), (64, 2048, 768, 128, 8, 0x40),
                # 'average' without a shared expert; no room for the shared expert
                (64, 2048, 768, 128, 8, 0x9), (64, 2048, 768, 1024, 8, 0x5),
                # W4A16 quantizes no activations: static scales do not apply
                (64, 2048, 768, 128, 8, 0x12), (64, 2048, 768, 128, 8, 0x20)]:
        c = binding.MoeConfig(*cfg)
        assert L.moe_workspace_create(ctypes.byref(c), None, ctypes.byref(h)) == 1, cfg
    assert L.moe_workspace_create(None, None, ctypes.byref(h)) == 1
    # calls on a NULL workspace fail before touching the device
    assert L.moe_nvfp4_forward(None, None, None, 1, None, None) == 1
    assert L.moe_nvfp4_forward_quantized(None, None, None, None, None, 1, None, None) == 1
    assert L.refresh_scales_inplace(None, None, None) == 1
    assert L.moe_workspace_bind_weights(None, None, None) == 1
    assert L.moe_pack_weights(None, None, None, None) == 1
    assert L.moe_workspace_destroy(None) == 0


def test_packed_bytes_host_only():
    """Packed unit-record sizes (host-only arithmetic, no device): four
    16-row fragments x 128-wide K steps x 4608-byte records, i.e. the NVFP4
    bytes of the matrix (0.5 + 1/16 B per element) exactly."""
    from nvfp4_token_quant_amd import binding
    for E, H, I in ((8, 256, 512), (128, 2048, 768), (256, 7168, 2048), (1, 128, 128)):
        b13, b2 = binding.packed_bytes(E, H, I)
        assert b13 == E * 2 * I * H * 9 // 16
        assert b2 == E * H * I * 9 // 16
        assert binding.packed_bytes(1, H, I) == (b13 // E, b2 // E)
    for bad in ((0, 256, 512), (8, 200, 512), (8, 256, 100), (2000, 256, 512)):
        with pytest.raises(binding.Nvfp4Error):
            binding.packed_bytes(*bad)
