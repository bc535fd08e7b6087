"""The helpers behind the GPU parity checks, pinned on the CPU: the bf16
storage allowance of an O delivered in bf16 is exactly the largest error of
round-to-nearest-even bf16 rounding, and case seeds do not depend on the
process."""

import numpy as np

from long_context_exact_amd.synth import bf16_round

from _util import bf16_half_spacing, case_seed


def test_half_spacing_bounds_and_is_attained_by_bf16_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 12, 200_000))).astype(np.float32)
    err = np.abs(bf16_round(x).astype(np.float64) - x.astype(np.float64))
    half = bf16_half_spacing(x)
    assert np.all(err <= half)
    assert float(np.max(err / half)) > 0.99  # ties and near-ties reach the bound


def test_half_spacing_exact_values():
    # bf16 keeps 8 significant bits: spacing 2**(e - 7) on [2**e, 2**(e + 1))
    x = np.array([1.0, 1.5, 2.0, 3.99, 4.0, 0.25, -6.0, 0.0])
    want = np.array([2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -10,
                     2.0 ** -6, 0.0])
    assert np.array_equal(bf16_half_spacing(x), want)


def test_case_seed_is_process_independent():
    assert case_seed((2, 300, "bf16")) == 2945852503
