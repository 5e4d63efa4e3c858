"""The bfloat16 output-rounding allowance used by the GPU parity tests,
checked against round-to-nearest-even itself (host code, no GPU)."""
import numpy as np

from exact_blockwise_attention_amd import synthetic as syn
from gpu_cases import bf16_half_spacing


def test_half_spacing_values():
    assert bf16_half_spacing(1.0) == 2.0 ** -8
    assert bf16_half_spacing(1.99) == 2.0 ** -8
    assert bf16_half_spacing(-9.87) == 2.0 ** -5
    assert bf16_half_spacing(0.0) == 0.0


def test_rounding_never_moves_a_value_more_than_half_a_spacing():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-10, 10, 200000))).astype(np.float32)
    r = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(x)).astype(np.float64)
    moved = np.abs(r - x.astype(np.float64))
    assert np.all(moved <= bf16_half_spacing(x))
    # the bound is attained: values half-way between neighbours move by it
    mid = np.float32(1.0 + 2.0 ** -8)
    r_mid = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(np.array([mid])))[0]
    assert abs(float(r_mid) - float(mid)) == bf16_half_spacing(float(mid))


def test_plain_bar_below_the_band():
    """Below |ref| = 4 a bf16 output gets the plain 2e-2 bar and nothing more."""
    import pytest

    from gpu_cases import assert_output_close
    ref = np.array([1.0, -3.9, 0.5])
    assert_output_close("x", ref + np.array([0.0199, -0.0199, 0.0]), ref, "bf16")
    with pytest.raises(AssertionError):
        assert_output_close("x", ref + np.array([0.0201, 0.0, 0.0]), ref, "bf16")
    with pytest.raises(AssertionError):  # 0.0201 would pass with the old allowance (half spacing 2^-7 at 3.9)
        assert_output_close("x", ref + np.array([0.0, -0.0201, 0.0]), ref, "bf16")


def test_rounding_allowance_only_in_the_band():
    """At |ref| >= 4 the half bf16 spacing of the output is added: the exact
    value 9.9 rounds to 9.875 (0.025 away), and 0.02 of arithmetic error on
    top of it passes, 0.05 does not."""
    import pytest

    from gpu_cases import assert_output_close
    ref = np.array([9.9, 1.0])
    got = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(np.array([9.9 + 0.02, 1.0], dtype=np.float32)))
    assert_output_close("x", got.astype(np.float64), ref, "bf16")
    with pytest.raises(AssertionError):
        assert_output_close("x", np.array([9.9 + 0.05 + 2.0 ** -5, 1.0]), ref, "bf16")
    # fp32 outputs never get the allowance
    with pytest.raises(AssertionError):
        assert_output_close("x", np.array([9.9 + 2e-4, 1.0]), ref, "f32")
