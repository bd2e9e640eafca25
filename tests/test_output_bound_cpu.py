"""The output bound of the GPU parity tests (gpu_common.output_bound), checked on the CPU.

The stated limits are absolute: 1e-2 on bf16 outputs, 2e-3 on fp16 outputs. Stored in a
16-bit format, an output of magnitude |O| can be off by half an ulp from rounding alone, and
that exceeds the stated limit from |O| = 4 (bf16: half an ulp is 2^-6 = 1.56e-2 in [4, 8))
and from |O| = 8 (fp16: half an ulp is 2^-8 = 3.9e-3 in [8, 16)). The bound keeps the stated limit
below those magnitudes and above them adds exactly the growth of the half-ulp. These checks
pin that: the stated limit is unchanged where it can be met, every correctly rounded output
passes at every magnitude, and an output one ulp beyond its correct rounding fails."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_common import TOL, output_bound, output_error

LIMIT = {"bf16": 4.0, "f16": 8.0}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}


def rounded(x: np.ndarray, dtype: str) -> np.ndarray:
    """x correctly rounded (to nearest, ties to even) to the storage format, as float64."""
    return torch.from_numpy(x).to(TORCH[dtype]).double().numpy()


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    p = {"bf16": 8, "f16": 11}[dtype]
    return np.exp2(np.floor(np.log2(np.abs(x))) - p + 1)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_the_stated_limit_holds_below_the_magnitude_where_it_can_be_met(dtype):
    to = TOL[dtype][0]
    rng = np.random.default_rng(1)
    O = rng.uniform(-LIMIT[dtype], LIMIT[dtype], 100000)
    o = rounded(O, dtype)
    keep = np.maximum(np.abs(o), np.abs(O)) < LIMIT[dtype]
    assert keep.mean() > 0.99
    assert (output_bound(o[keep], O[keep], dtype, to) == to).all()
    # and half an ulp, the most a correct rounding costs, fits inside it there
    assert np.abs(o[keep] - O[keep]).max() <= to


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_above_it_the_bound_grows_by_the_half_ulp(dtype):
    to = TOL[dtype][0]
    L = LIMIT[dtype]
    half_below = float(ulp(np.array([L / 2]), dtype)[0]) / 2     # half an ulp just below L
    for k in range(0, 5):
        x = np.array([L * 2 ** k * 1.25])
        half = float(ulp(x, dtype)[0]) / 2
        assert float(output_bound(x, x, dtype, to)[0]) == pytest.approx(to + half - half_below)
    assert float(output_bound(np.array([5.0]), np.array([5.0]), "bf16", 1e-2)[0]) == \
        pytest.approx(1e-2 + 2 ** -6 - 2 ** -7)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_every_correctly_rounded_output_passes(dtype):
    to = TOL[dtype][0]
    rng = np.random.default_rng(2)
    O = np.concatenate([rng.standard_normal(200000) * 6, rng.uniform(-200, 200, 50000),
                        np.array([3.999, 4.0, 4.001, 7.999, 8.0, 8.001, -3.9999, -4.0, 0.0])])
    o = rounded(O, dtype)
    err, excess, _ = output_error(o, O, dtype, to)
    assert excess <= 0
    assert err > to if dtype == "bf16" else True     # the stated limit alone would fail these


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_one_ulp_beyond_the_correct_rounding_fails(dtype):
    to = TOL[dtype][0]
    rng = np.random.default_rng(3)
    for lo, hi in [(LIMIT[dtype], 2 * LIMIT[dtype]), (2 * LIMIT[dtype], 8 * LIMIT[dtype])]:
        O = rng.uniform(lo, hi, 2000)
        o = rounded(O, dtype)
        o_bad = o + ulp(o, dtype) * np.sign(o - O + 1e-300)   # one step further from O
        _, excess, _ = output_error(o_bad, O, dtype, to)
        assert excess > 0
    # below the limit the stated limit itself applies
    O = np.array([1.0])
    _, excess, at = output_error(O + 1.01 * to, O, dtype, to)
    assert excess > 0 and at == 1.0


def test_non_finite_outputs_fail():
    with pytest.raises(AssertionError):
        output_error(np.array([np.inf]), np.array([1.0]), "bf16", 1e-2)
