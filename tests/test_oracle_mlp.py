"""Pins for the oracle's MLP (CPU).

Closed forms and textbook values: silu(0) = 0, sigmoid(0) = 1/2, the odd
part silu(z) - silu(-z) = z, textbook sigmoid values, group-size invariance
when all groups of a row share (scale, bias), constant weights, x = 0 gives
y = r, the residual shifts y one for one, ffn permutation invariance, a
hand-derived tiny MLP (tests/golden/mlp_tiny_hand.json), and a brute-force
exact-rational implementation on tiny random inputs."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import load_golden
from workloads import generic_weights


# ------------------------------------------------------------------ silu

def test_silu_zero_and_half():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    z = np.array([1e-12, -1e-12])
    assert np.allclose(oracle.silu(z) / z, 0.5, rtol=1e-9)     # sigmoid(0) = 1/2


def test_silu_textbook():
    t = load_golden("sigmoid_textbook.json")
    got = oracle.silu(np.array(t["z"]))
    assert np.allclose(got, t["silu"], rtol=1e-15, atol=1e-300)


def test_silu_odd_part():
    z = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)


def test_silu_tails_do_not_overflow():
    with np.errstate(over="raise", invalid="raise"):
        big = oracle.silu(np.array([1000.0, -1000.0, 745.0, -745.0]))
    assert big[0] == 1000.0 and big[2] == 745.0
    assert big[1] == 0.0 and abs(big[3]) < 1e-300


# ------------------------------------------------------------------ gemv parts

@pytest.mark.parametrize("bits", [4, 8])
def test_group_size_invariance(bits):
    """If every group of a row shares (s, b), W~x = s*(Q x) + b*sum(x) for any g."""
    rng = np.random.default_rng(7)
    k, n = 256, 6
    q = rng.integers(0, 1 << bits, size=(n, k), dtype=np.uint8)
    x = rng.integers(-8, 9, size=(1, k)).astype(np.float64)      # exact in fp64
    s_row = np.array([2.0 ** -e for e in range(1, n + 1)], dtype=np.float32)
    b_row = np.array([-0.5, 0.25, 1.0, -2.0, 0.0, 0.125], dtype=np.float32)
    closed = s_row[:, None] * (q.astype(np.int64) @ x[0].astype(np.int64))[:, None] \
        + b_row[:, None] * x.sum()
    outs = []
    for g in (32, 64, 128):
        s = np.repeat(s_row[:, None], k // g, axis=1)
        b = np.repeat(b_row[:, None], k // g, axis=1)
        w = oracle.dequantize(q, s, b, g)
        gg, _, _ = oracle.gate_up_swiglu(x, w, w)
        outs.append(gg[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert np.array_equal(outs[0], closed[:, 0])


def test_constant_weights():
    """W~ = c everywhere (constant groups: scale 0, bias c) gives c * sum(x)."""
    x = np.array([[0.5, -1.25, 2.0, 3.0] * 8])
    w = np.full((3, 32), np.float32(0.75))
    q, s, b = oracle.quantize_affine(w.astype(np.float32), 8, 32)
    wt = oracle.dequantize(q, s, b, 32)
    g, u, h = oracle.gate_up_swiglu(x, wt, 2 * wt)
    assert np.all(g == 0.75 * x.sum()) and np.all(u == 1.5 * x.sum())


def test_gate_and_up_are_not_interchangeable():
    """g = 2, u = 3 gives h = 3 * silu(2); the swapped epilogue would give 2 * silu(3)."""
    t = load_golden("sigmoid_textbook.json")
    x = np.ones((1, 32))
    wg = np.full((1, 32), 2.0 / 32)
    wu = np.full((1, 32), 3.0 / 32)
    g, u, h = oracle.gate_up_swiglu(x, wg, wu)
    assert g[0, 0] == 2.0 and u[0, 0] == 3.0
    assert h[0, 0] == pytest.approx(3 * t["silu"][4], rel=1e-15)


def test_hand_tiny_mlp():
    t = load_golden("mlp_tiny_hand.json")
    d, ffn = t["d"], t["ffn"]
    x = np.ones((1, d)); x[0, 0] = 2; x[0, 31] = -1
    gq = np.zeros((ffn, d), np.uint8); gq[0] = np.arange(d)
    gs = np.array([[1 / 64], [0]], np.float32); gb = np.array([[-0.25], [0]], np.float32)
    uq = np.zeros((ffn, d), np.uint8); uq[1] = 255
    us = np.array([[0], [1 / 256]], np.float32); ub = np.array([[0.5], [0]], np.float32)
    dq = np.zeros((d, ffn), np.uint8); dq[:, 0] = np.arange(d); dq[:, 1] = 7
    ds = np.full((d, 1), 1 / 16, np.float32); db = np.zeros((d, 1), np.float32)
    r = (np.arange(d) / 32.0)[None, :]
    wg = oracle.dequantize(gq, gs, gb, t["gate_group"])
    wu = oracle.dequantize(uq, us, ub, t["gate_group"])
    wd = oracle.dequantize(dq, ds, db, t["down_group"])
    g, u, h = oracle.gate_up_swiglu(x, wg, wu)
    assert g[0].tolist() == t["g"] and u[0].tolist() == t["u"]
    assert h[0] == pytest.approx(t["h"], rel=1e-15)
    h2, y = oracle.mlp_decode(x, r, wg, wu, wd)
    expect = np.arange(d) / 32.0 + np.arange(d) / 16.0 * t["h0"]
    assert np.allclose(y[0], expect, rtol=1e-15, atol=1e-15)


def test_down_orientation_nonsquare():
    """W_down is [d, ffn]: y_i = r_i + sum_n W[i, n] h_n (a transposed operand fails)."""
    h = np.array([[1.0, 10.0, 100.0]])
    wd = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    r = np.array([[0.5, -0.5]])
    y = oracle.down_residual(h, r, wd)
    assert y.tolist() == [[321.5, 653.5]]
    with pytest.raises(ValueError):
        oracle.down_residual(h, r, wd.T)


# ------------------------------------------------------------------ whole MLP

def _random_mlp(seed, d=64, ffn=96, m=2, group=32, bits=8):
    wg = generic_weights((seed, 1), ffn, d, 0.05)
    wu = generic_weights((seed, 2), ffn, d, 0.05)
    wd = generic_weights((seed, 3), d, ffn, 0.05)
    deq = []
    for w in (wg, wu, wd):
        q, s, b = oracle.quantize_affine(w, bits, group)
        deq.append(oracle.dequantize(q, s, b, group))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, d))
    r = rng.standard_normal((m, d))
    return x, r, deq


def test_zero_input_gives_residual():
    x, r, (wg, wu, wd) = _random_mlp(1)
    h, y = oracle.mlp_decode(np.zeros_like(x), r, wg, wu, wd)
    assert np.all(h == 0) and np.array_equal(y, r)


def test_zero_down_gives_residual():
    x, r, (wg, wu, wd) = _random_mlp(2)
    h, y = oracle.mlp_decode(x, r, wg, wu, np.zeros_like(wd))
    assert np.array_equal(y, r)


def test_residual_shift():
    x, r, (wg, wu, wd) = _random_mlp(3)
    delta = np.linspace(-1, 1, r.size).reshape(r.shape)
    _, y0 = oracle.mlp_decode(x, r, wg, wu, wd)
    _, y1 = oracle.mlp_decode(x, r + delta, wg, wu, wd)
    assert np.allclose(y1 - y0, delta, atol=1e-12)


def test_ffn_permutation_invariance():
    x, r, (wg, wu, wd) = _random_mlp(4)
    p = np.random.default_rng(9).permutation(wg.shape[0])
    _, y0 = oracle.mlp_decode(x, r, wg, wu, wd)
    _, y1 = oracle.mlp_decode(x, r, wg[p], wu[p], wd[:, p])
    assert np.allclose(y0, y1, rtol=1e-13, atol=1e-13)


def test_rows_are_independent():
    x, r, (wg, wu, wd) = _random_mlp(5, m=3)
    _, y = oracle.mlp_decode(x, r, wg, wu, wd)
    for i in range(3):
        _, yi = oracle.mlp_decode(x[i:i + 1], r[i:i + 1], wg, wu, wd)
        assert np.allclose(yi[0], y[i], rtol=1e-14, atol=1e-14)


def _silu_exact_ish(z: Fraction) -> float:
    zf = float(z)
    return zf / (1.0 + math.exp(-zf)) if zf >= 0 else zf * math.exp(zf) / (1.0 + math.exp(zf))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_rational(seed):
    """Quantize, dequantize and both projections in exact rationals with plain
    loops (silu via math.exp), against the vectorized oracle."""
    d, ffn, group, bits = 8, 4, 4, 8
    rng = np.random.default_rng(100 + seed)
    wg = (rng.standard_normal((ffn, d)) * 0.3).astype(np.float32)
    wu = (rng.standard_normal((ffn, d)) * 0.3).astype(np.float32)
    wd = (rng.standard_normal((d, ffn)) * 0.3).astype(np.float32)
    x = rng.standard_normal(d).astype(np.float32)
    r = rng.standard_normal(d).astype(np.float32)

    def quant_exact(w):
        """Rational quantizer with the same reading: the scale is the fp32
        nearest to span/qmax; codes round half to even."""
        qmax = (1 << bits) - 1
        rows = []
        for i in range(w.shape[0]):
            row = []
            for j in range(0, w.shape[1], group):
                vals = [Fraction(float(v)) for v in w[i, j:j + group]]
                mn, mx = min(vals), max(vals)
                scale = Fraction(float(np.float32(float((mx - mn) / qmax))))
                for v in vals:
                    if scale == 0:
                        row.append(mn)
                        continue
                    t = (v - mn) / scale
                    fl = t.numerator // t.denominator
                    frac = t - fl
                    q = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2) else 0)
                    q = min(max(q, 0), qmax)
                    row.append(scale * q + mn)
            rows.append(row)
        return rows

    WG, WU, WD = quant_exact(wg), quant_exact(wu), quant_exact(wd)
    X = [Fraction(float(v)) for v in x]
    hs = []
    for n in range(ffn):
        g = sum(WG[n][k] * X[k] for k in range(d))
        u = sum(WU[n][k] * X[k] for k in range(d))
        hs.append(_silu_exact_ish(g) * float(u))
    y_bf = [float(r[i]) + float(sum(WD[i][n] * Fraction(hs[n]) for n in range(ffn)))
            for i in range(d)]

    deq = []
    for w in (wg, wu, wd):
        q, s, b = oracle.quantize_affine(w, bits, group)
        deq.append(oracle.dequantize(q, s, b, group))
    h, y = oracle.mlp_decode(x[None, :], r[None, :], *deq)
    assert np.allclose(h[0], hs, rtol=1e-12, atol=1e-14)
    assert np.allclose(y[0], y_bf, rtol=1e-12, atol=1e-14)


def test_dense_is_textbook_matmul():
    rng = np.random.default_rng(11)
    bits_g = rng.integers(0x3C00, 0x3D00, size=(5, 16)).astype(np.uint16)
    bits_u = rng.integers(0xBC00, 0xBD00, size=(5, 16)).astype(np.uint16)
    wg = oracle.dequantize_dense_bf16(bits_g)
    wu = oracle.dequantize_dense_bf16(bits_u)
    x = rng.standard_normal((1, 16))
    g, u, h = oracle.gate_up_swiglu(x, wg, wu)
    for n in range(5):
        assert g[0, n] == pytest.approx(sum(wg[n, k] * x[0, k] for k in range(16)), rel=1e-14)
        assert u[0, n] == pytest.approx(sum(wu[n, k] * x[0, k] for k in range(16)), rel=1e-14)
