"""Pins for the oracle's MXFP4 / MXFP8 (CPU): element and scale values from
the format definitions, exact round trips, ties and saturation worked by
hand, the zero block and negative zero, a brute-force quantizer that picks
the nearest grid value by enumeration, the error bound, and the nibble
order of the stored bytes."""
import math

import numpy as np
import pytest

import oracle


def test_e2m1_values():
    assert oracle.decode_element(np.arange(8), "mxfp4").tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert oracle.decode_element(np.arange(9, 16), "mxfp4").tolist() == [-0.5, -1, -1.5, -2, -3, -4, -6]


def test_e4m3_values():
    d = oracle.decode_element(np.arange(256), "mxfp8")
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x7E] == 448.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x3C] == 1.5 and d[0x40] == 2.0 and d[0x30] == 0.5
    assert math.isnan(d[0x7F]) and math.isnan(d[0xFF])
    fin = d[:0x7F]
    assert np.all(np.diff(fin) > 0)              # magnitudes strictly increase with the code


def test_scale_values():
    assert oracle.decode_scale([127, 128, 0, 254]).tolist() == [1.0, 2.0, 2.0 ** -127, 2.0 ** 127]


@pytest.mark.parametrize("fmt,top", [("mxfp4", 6.0), ("mxfp8", 448.0)])
def test_exact_round_trip(fmt, top):
    grid = np.unique(np.abs(oracle.decode_element(np.arange(16 if fmt == "mxfp4" else 127), fmt)))
    rng = np.random.default_rng(1)
    vals = rng.choice(grid, size=(3, 32)) * rng.choice([-1.0, 1.0], size=(3, 32))
    vals[:, 0] = top                                  # pins the shared exponent at 2^0
    for s in (0, 5, -9):
        w = vals * 2.0 ** s
        c, e = oracle.quantize_mx(w, fmt)
        assert np.all(e == 127 + s)
        assert np.array_equal(oracle.dequantize_mx(c, e, fmt), w)


def test_hand_cases_e2m1():
    w = np.zeros((1, 32))
    w[0, :8] = [6.0, 2.5, 3.5, 5.0, 7.5, -0.2, 0.25, 0.75]
    c, e = oracle.quantize_mx(w, "mxfp4")
    assert e[0, 0] == 127                         # floor(log2 7.5) - 2 = 0
    d = oracle.decode_element(c[0, :8], "mxfp4")
    # 2.5 -> 2 and 3.5 -> 4 and 5 -> 4 (ties to the even mantissa), 7.5 saturates at 6,
    # -0.2 -> -0 (sign kept), 0.25 -> 0 (tie to even), 0.75 -> 1 (tie between 0.5 and 1: even is 1)
    assert d.tolist() == [6.0, 2.0, 4.0, 4.0, 6.0, -0.0, 0.0, 1.0]
    assert c[0, 5] == 8


def test_hand_cases_e4m3():
    w = np.zeros((1, 32))
    w[0, :4] = [256.0, 1.0 + 1 / 16, 1.0 + 3 / 16, 500.0]
    c, e = oracle.quantize_mx(w, "mxfp8")
    assert e[0, 0] == 127 + 8 - 8                 # floor(log2 500) = 8, minus 8
    assert oracle.decode_element(c[0, :4], "mxfp8").tolist() == [256.0, 1.0, 1.25, 448.0]


def test_zero_block_and_scale_range():
    c, e = oracle.quantize_mx(np.zeros((2, 64)), "mxfp8")
    assert np.all(c == 0) and np.all(e == 0)
    c, e = oracle.quantize_mx(np.full((1, 32), 2.0 ** -140), "mxfp4")   # shared exponent clamps at -127
    assert e[0, 0] == 0


def _brute(block, fmt):
    """Nearest grid value by enumeration; ties to the even code."""
    n_codes = 8 if fmt == "mxfp4" else 127
    grid = oracle.decode_element(np.arange(n_codes), fmt)
    emax = 2 if fmt == "mxfp4" else 8
    amax = max(abs(v) for v in block)
    if amax == 0:
        return [0] * 32, 0
    shared = max(-127, min(127, math.floor(math.log2(amax)) - emax))
    x = 2.0 ** shared
    codes = []
    for v in block:
        t = abs(v) / x
        best = None
        for cd in range(n_codes):
            dist = abs(grid[cd] - t)
            if best is None or dist < best[0] or (dist == best[0] and cd % 2 == 0):
                best = (dist, cd)
        cd = best[1] if t <= grid[-1] else n_codes - 1
        sign = 8 if fmt == "mxfp4" else 128
        codes.append(cd | (sign if v < 0 else 0))
    return codes, shared + 127


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_brute_force(fmt):
    rng = np.random.default_rng(7)
    w = rng.normal(0, 0.02, size=(6, 64)) * np.exp(rng.normal(0, 2, size=(6, 64)))
    c, e = oracle.quantize_mx(w, fmt)
    for r in range(6):
        for b in range(2):
            bc, be = _brute(w[r, 32 * b:32 * b + 32].tolist(), fmt)
            assert e[r, b] == be
            assert c[r, 32 * b:32 * b + 32].tolist() == bc


@pytest.mark.parametrize("fmt,mb", [("mxfp4", 1), ("mxfp8", 3)])
def test_error_bound(fmt, mb):
    """Unsaturated values land within half a grid step of the scaled element."""
    rng = np.random.default_rng(8)
    w = rng.normal(size=(16, 256))
    c, e = oracle.quantize_mx(w, fmt)
    deq = oracle.dequantize_mx(c, e, fmt)
    x = np.repeat(oracle.decode_scale(e), 32, axis=1)
    t = np.abs(w) / x
    top = 6.0 if fmt == "mxfp4" else 448.0
    ok = t <= top
    emin = 0 if fmt == "mxfp4" else -6
    step = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.maximum(t, 1e-300))), emin).astype(int) - mb) * x
    assert np.all(np.abs(w - deq)[ok] <= step[ok] / 2 * (1 + 1e-12))


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    assert oracle.pack_mx_codes(codes, "mxfp4").tolist() == [[0x21, 0x43, 0x0F]]
    assert oracle.pack_mx_codes(codes, "mxfp8").tolist() == codes.tolist()
