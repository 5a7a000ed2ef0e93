"""Pins for the oracle's projection y = x W^T + b (CPU): x = 0 gives the bias,
a one-hot x selects a column of W plus the bias (which fixes the
orientation), a hand-computed non-square case, and a loop implementation on
tiny inputs."""
import numpy as np
import pytest

import oracle


def test_zero_input_gives_bias():
    rng = np.random.default_rng(1)
    w, b = rng.normal(size=(7, 5)), rng.normal(size=7)
    y = oracle.linear(np.zeros((3, 5)), w, b)
    assert np.array_equal(y, np.tile(b, (3, 1)))
    assert np.array_equal(oracle.linear(np.zeros((1, 5)), w), np.zeros((1, 7)))


@pytest.mark.parametrize("j", [0, 2, 4])
def test_one_hot_selects_a_column(j):
    rng = np.random.default_rng(2)
    w, b = rng.normal(size=(6, 5)), rng.normal(size=6)
    x = np.zeros(5)
    x[j] = 1.0
    assert np.array_equal(oracle.linear(x, w, b)[0], w[:, j] + b)


def test_hand_case():
    w = np.array([[1.0, 2.0, 3.0], [-1.0, 0.5, 0.0]])       # n = 2, k = 3
    x = np.array([[2.0, -1.0, 4.0]])
    y = oracle.linear(x, w, np.array([0.25, -2.0]))
    assert y.tolist() == [[2.0 - 2.0 + 12.0 + 0.25, -2.0 - 0.5 + 0.0 - 2.0]]


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    w, x, b = rng.normal(size=(4, 6)), rng.normal(size=(2, 6)), rng.normal(size=4)
    y = oracle.linear(x, w, b)
    for i in range(2):
        for n in range(4):
            acc = b[n]
            for k in range(6):
                acc += x[i, k] * w[n, k]
            assert abs(y[i, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.linear(np.zeros((1, 4)), np.zeros((3, 5)))
    with pytest.raises(ValueError):
        oracle.linear(np.zeros((1, 5)), np.zeros((3, 5)), np.zeros(4))
