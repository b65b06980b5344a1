"""The layer tolerance's bf16 rounding term, pinned against the spacing of
bf16 values taken from their bit patterns (the next pattern up minus the
value), and the tolerance check on outputs that are the exact reference
rounded to bf16 (which must pass at any magnitude) or off by one bf16 step
more than the bound (which must fail)."""
import numpy as np
import pytest

from nvfp4_token_quant_amd import synth
from tests.layer_fixtures import bf16_half_ulp, check_layer_tolerance


def test_half_ulp_is_half_the_bf16_spacing():
    bits = np.arange(0x0080, 0x7F7F, 7, dtype=np.uint16)          # positive normal bf16 values
    v = synth.bf16_to_f32(bits).astype(np.float64)
    nxt = synth.bf16_to_f32(bits + 1).astype(np.float64)
    # a value strictly inside [v, next) has the same spacing as v
    inside = v + (nxt - v) * 0.3
    np.testing.assert_array_equal(bf16_half_ulp(inside), (nxt - v) / 2)
    np.testing.assert_array_equal(bf16_half_ulp(-inside), (nxt - v) / 2)


def test_tolerance_accepts_bf16_rounding_of_large_outputs():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(200000)
    ref[:50] *= 12.0                                              # outputs far in the tail
    got = synth.bf16_to_f32(synth.bf16_bits(ref.astype(np.float32))).astype(np.float64)
    raw = np.abs(got - ref).max() / np.sqrt((ref ** 2).mean())
    assert raw > 3e-2                                             # the raw max bound alone would fail
    check_layer_tolerance(got, ref)
    bad = got.copy()
    bad[7] = ref[7] + 0.05 * np.sqrt((ref ** 2).mean()) + 2 * bf16_half_ulp(ref[7])
    with pytest.raises(AssertionError):
        check_layer_tolerance(bad, ref)
