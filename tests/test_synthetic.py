"""The seeded input generator: bf16 round-to-nearest-even and reproducibility."""
import numpy as np

import synthetic as syn


def test_bf16_rne_halfway_cases():
    one = 1.0
    ulp = 2.0 ** -7          # bf16 spacing in [1, 2)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -20, -(one + ulp / 2),
                  3.0e38, 1e-40], dtype=np.float32)
    got = syn.bf16_bits_to_f32(syn.bf16_bits_from_f32(x))
    assert got[0] == one
    assert got[1] == one                      # tie -> even (mantissa 0)
    assert got[2] == one + 2 * ulp            # tie -> even (rounds up)
    assert got[3] == one + ulp                # above the tie rounds up
    assert got[4] == -one
    assert got[5] == np.float32(3.0e38) or abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8
    assert got[6] >= 0


def test_bf16_roundtrip_exact_values():
    v = np.arange(-256, 257, dtype=np.float32)
    assert np.array_equal(syn.bf16_bits_to_f32(syn.bf16_bits_from_f32(v)), v)


def test_seeded_draws_reproducible_and_scaled():
    a = syn.normal(7, (256, 512), 0.02, syn.BF16)
    b = syn.normal(7, (256, 512), 0.02, syn.BF16)
    assert np.array_equal(a.raw, b.raw)
    assert abs(float(a.f64.std()) - 0.02) < 0.001
    t = syn.targets(3, 10000, 151936)
    assert t.dtype == np.int32 and t.min() >= 0 and t.max() < 151936
