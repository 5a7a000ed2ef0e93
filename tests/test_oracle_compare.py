"""Pins of the comparator every parity assertion goes through.

The meTile "Compute-Graph Fusion" page (section "Automatic Gated Epilogues")
gates generated reductions by a scale-normalized primitive error; the reading
here is the largest absolute difference over all elements divided by the
largest absolute reference value.  Each case below is worked by hand and is
chosen so that a plausible slip fails it: a mean instead of a max, the output
instead of the reference as the scale, a per-row instead of a global maximum,
a dropped absolute value, a NaN that compares as small."""
import math

import numpy as np
import pytest

from oracle import scaled_error


def test_hand_value():
    # differences 0, 0, 1; largest |ref| 4
    assert scaled_error([1.0, 2.0, 3.0], [1.0, 2.0, 4.0]) == 0.25


def test_signs_use_absolute_values():
    # |(-1) - 1| = 2, |3 - (-4)| = 7; largest |ref| = 4 (from -4)
    assert scaled_error([-1.0, 3.0], [1.0, -4.0]) == 1.75
    # a negative difference counts by its size
    assert scaled_error([0.0, -3.0], [0.0, 2.0]) == 2.5


def test_scale_is_the_reference_not_the_output():
    # by max|out| this would be 0.5
    assert scaled_error([0.0, 10.0], [0.0, 5.0]) == 1.0


def test_max_not_mean():
    # the mean difference would be 1, the max is 4
    assert scaled_error([1.0, 1.0, 1.0, 5.0], [1.0, 1.0, 1.0, 1.0]) == 4.0
    # the mean |ref| would be 1.75, the max is 4
    assert scaled_error([2.0, 1.0, 1.0, 4.0], [1.0, 1.0, 1.0, 4.0]) == 0.25


def test_global_over_all_elements():
    # per-row maxima would give 0.5 for the first row
    out = np.array([[1.0, 0.0], [0.0, 10.0]])
    ref = np.array([[2.0, 0.0], [0.0, 10.0]])
    assert scaled_error(out, ref) == 1.0 / 10.0


def test_zero_reference():
    assert scaled_error([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert scaled_error([0.0, -0.0], [0.0, 0.0]) == 0.0
    assert scaled_error([0.0, 1e-30], [0.0, 0.0]) == math.inf


def test_empty_is_zero():
    assert scaled_error(np.zeros(0), np.zeros(0)) == 0.0


def test_nan_never_passes_a_tolerance():
    e = scaled_error([math.nan, 1.0], [1.0, 1.0])
    assert not (e <= 1.0)
    e = scaled_error([1.0, math.inf], [1.0, 1.0])
    assert not (e <= 1e300)


def test_shape_mismatch_raises():
    with pytest.raises(ValueError):
        scaled_error([1.0, 2.0], [1.0, 2.0, 3.0])
    with pytest.raises(ValueError):
        scaled_error(np.zeros((2, 3)), np.zeros((3, 2)))


def test_exact_in_fp64_for_narrow_inputs():
    # fp32 / bf16 outputs are widened exactly: 1 + 2^-23 against 1 gives 2^-23
    out = np.array([1.0 + 2.0 ** -23], dtype=np.float32)
    assert scaled_error(out, [1.0]) == 2.0 ** -23
