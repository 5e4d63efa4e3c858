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
