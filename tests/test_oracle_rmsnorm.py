"""Pins for the oracle's residual add + RMSNorm (CPU): hand cases
(tests/golden/rmsnorm_hand.json), the constant-vector closed form (which
also fixes where eps sits), s = 0, unit weights, and dtype rounding ties."""
import math

import numpy as np
import pytest

import oracle
from conftest import load_golden


@pytest.mark.parametrize("case", load_golden("rmsnorm_hand.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case):
    s, n = oracle.add_rmsnorm(np.array([case["a"]]), np.array([case["b"]]),
                              np.array(case["w"]), case["eps"], case["dtype"])
    assert s[0].tolist() == case["s"]
    if "n" in case:
        assert np.allclose(n[0], case["n"], rtol=1e-15)


@pytest.mark.parametrize("c", [1.0, -2.5, 0.003, 1e-3])
def test_constant_vector(c):
    """s = c*1: n = c*w/sqrt(c^2 + eps).  With c^2 near eps the placement of
    eps (inside the root) and of w (after normalizing) both matter."""
    n_el, eps = 64, 1e-5
    w = np.linspace(0.5, 1.5, n_el)
    s, n = oracle.add_rmsnorm(np.full((1, n_el), c), np.zeros((1, n_el)), w, eps, "f32")
    cf = float(np.float32(c))
    expect = cf * w / math.sqrt(cf * cf + eps)
    assert np.allclose(n[0], expect, rtol=1e-14)


def test_zero_vector():
    s, n = oracle.add_rmsnorm(np.zeros((2, 16)), np.zeros((2, 16)), np.ones(16), 1e-5, "f16")
    assert np.all(s == 0) and np.all(n == 0)


def test_unit_weight_mean_square():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((3, 256)).astype(np.float32)
    b = rng.standard_normal((3, 256)).astype(np.float32)
    eps = 1e-5
    s, n = oracle.add_rmsnorm(a, b, np.ones(256), eps, "f32")
    ms = np.mean(s * s, axis=1)
    assert np.allclose(np.mean(n * n, axis=1), ms / (ms + eps), rtol=1e-13)


def test_rows_independent():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((4, 32))
    b = rng.standard_normal((4, 32))
    w = rng.uniform(0.5, 1.5, 32)
    s, n = oracle.add_rmsnorm(a, b, w, 1e-5, "f32")
    s1, n1 = oracle.add_rmsnorm(a[2:3], b[2:3], w, 1e-5, "f32")
    assert np.array_equal(s[2], s1[0]) and np.array_equal(n[2], n1[0])


def test_round_to_dtype_matches_storage_types():
    """f32 / f16 rounding agree with numpy's casts; bf16 agrees with keeping the
    top 16 bits after nearest-even rounding, on random and tie values."""
    rng = np.random.default_rng(8)
    v = rng.standard_normal(4096) * np.exp(rng.uniform(-20, 20, 4096))
    assert np.array_equal(oracle.round_to_dtype(v, "f32"), v.astype(np.float32).astype(np.float64))
    vs = v[np.abs(v) < 60000]
    assert np.array_equal(oracle.round_to_dtype(vs, "f16"), vs.astype(np.float16).astype(np.float64))
    # bf16 ties: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6, and sign symmetry
    t = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3 * 2 ** -134])
    assert oracle.round_to_dtype(t, "bf16").tolist() == [1.0, 1 + 2 ** -6, -1.0, 2 ** -130, 2 ** -132]
    # every rounded value is a bf16: its fp32 image has 16 zero low bits
    r = oracle.round_to_dtype(v[np.abs(v) < 1e38], "bf16").astype(np.float32)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # and it is the nearest one: no bf16 neighbour is closer
    up = (r.view(np.uint32) + (1 << 16)).view(np.float32).astype(np.float64)
    dn = (r.view(np.uint32) - (1 << 16)).view(np.float32).astype(np.float64)
    vv = v[np.abs(v) < 1e38]
    rr = r.astype(np.float64)
    assert np.all(np.abs(vv - rr) <= np.abs(vv - up)) and np.all(np.abs(vv - rr) <= np.abs(vv - dn))
