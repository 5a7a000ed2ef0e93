"""Pins for the oracle's decode chain (CPU): a brute-force loop
implementation on tiny inputs (f32 and f16 rounding through struct), the
zero-weight special cases (y is the rounded sum, not a), RMSNorm's scale
invariance carried through the MLP, and the constant-vector closed form."""
import math
import struct

import numpy as np
import pytest

import oracle


def _round(v, dtype):
    fmt = {"f32": "f", "f16": "e"}[dtype]
    return struct.unpack(fmt, struct.pack(fmt, v))[0]


def _brute(a, b, w, eps, dtype, wg, wu, wd):
    d, ffn = len(a), len(wg)
    s = [_round(a[i] + b[i], dtype) for i in range(d)]
    ms = 0.0
    for v in s:
        ms += v * v
    ms /= d
    x = [_round(s[i] / math.sqrt(ms + eps) * w[i], dtype) for i in range(d)]
    h = []
    for f in range(ffn):
        g = u = 0.0
        for i in range(d):
            g += wg[f][i] * x[i]
            u += wu[f][i] * x[i]
        h.append(g / (1.0 + math.exp(-g)) * u)
    y = []
    for i in range(d):
        acc = 0.0
        for f in range(ffn):
            acc += wd[i][f] * h[f]
        y.append(s[i] + acc)
    return s, x, h, y


def _tiny(seed, dtype, d=5, ffn=3):
    rng = np.random.default_rng(seed)
    def q(v):
        return np.array([_round(float(t), dtype) for t in np.ravel(v)]).reshape(np.shape(v))
    a, b = q(rng.normal(size=d)), q(rng.normal(size=d))
    w = q(rng.uniform(0.5, 1.5, size=d))
    wg, wu = rng.normal(0, 0.5, (ffn, d)), rng.normal(0, 0.5, (ffn, d))
    wd = rng.normal(0, 0.5, (d, ffn))
    return a, b, w, wg, wu, wd


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_tiny(dtype, seed):
    a, b, w, wg, wu, wd = _tiny(seed, dtype)
    eps = 1e-5
    s, x, h, y = oracle.mlp_decode_rmsnorm(a[None], b[None], w, eps, dtype, wg, wu, wd)
    bs, bx, bh, by = _brute(a.tolist(), b.tolist(), w.tolist(), eps, dtype, wg.tolist(), wu.tolist(), wd.tolist())
    assert s[0].tolist() == bs
    assert x[0].tolist() == bx
    assert np.allclose(h[0], bh, rtol=1e-12, atol=1e-15)
    assert np.allclose(y[0], by, rtol=1e-12, atol=1e-15)


def test_zero_norm_weight_gives_the_sum():
    """w = 0 makes the MLP input 0, so h = silu(0) * 0 = 0 and y = s exactly."""
    a, b, _, wg, wu, wd = _tiny(7, "f32", d=16, ffn=8)
    s, x, h, y = oracle.mlp_decode_rmsnorm(a[None], b[None], np.zeros(16), 1e-5, "f32", wg, wu, wd)
    assert np.all(x == 0) and np.all(h == 0)
    assert np.array_equal(y, s)


def test_zero_mlp_gives_rounded_sum_not_a():
    """With all MLP weights zero the output is the residual: round(a + b)."""
    rng = np.random.default_rng(8)
    a = oracle.round_to_dtype(rng.normal(size=(1, 32)), "bf16")
    b = oracle.round_to_dtype(rng.normal(size=(1, 32)), "bf16")
    w = np.ones(32)
    z1, z2 = np.zeros((16, 32)), np.zeros((32, 16))
    s, _, _, y = oracle.mlp_decode_rmsnorm(a, b, w, 1e-5, "bf16", z1, z1, z2)
    assert np.array_equal(y, oracle.round_to_dtype(a + b, "bf16"))
    assert not np.array_equal(y, a)


def test_scale_invariance():
    """With eps = 0, scaling a and b by 2^3 scales s exactly and leaves the
    normalized row, h, and y - s unchanged."""
    a, b, w, wg, wu, wd = _tiny(9, "f32", d=24, ffn=10)
    s1, x1, h1, y1 = oracle.mlp_decode_rmsnorm(a[None], b[None], w, 0.0, "f32", wg, wu, wd)
    s2, x2, h2, y2 = oracle.mlp_decode_rmsnorm(8 * a[None], 8 * b[None], w, 0.0, "f32", wg, wu, wd)
    assert np.array_equal(s2, 8 * s1)
    assert np.array_equal(x2, x1) and np.array_equal(h2, h1)
    assert np.allclose(y2 - s2, y1 - s1, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("c", [0.75, -3.0])
def test_constant_vector(c):
    """s = c * 1 with eps = 0 normalizes to sign(c) * w exactly, so the chain
    is the MLP on sign(c) * w with residual s."""
    d = 32
    _, _, _, wg, wu, wd = _tiny(10, "f32", d=d, ffn=12)
    w = np.linspace(0.5, 1.5, d)
    w = np.array([_round(float(t), "f32") for t in w])
    s, x, h, y = oracle.mlp_decode_rmsnorm(np.full((1, d), c), np.zeros((1, d)), w, 0.0, "f32", wg, wu, wd)
    assert np.array_equal(x[0], math.copysign(1.0, c) * w)
    _, y_ref = oracle.mlp_decode(math.copysign(1.0, c) * w[None], s, wg, wu, wd)
    assert np.array_equal(y, y_ref)
