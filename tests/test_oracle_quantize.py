"""Pins for the oracle's affine quantizer and dequantizer (CPU).

The quantizer is an encoding, so it is pinned by hand-built groups whose
codes follow from the formula by hand (tests/golden/quantize_hand.json),
by properties every correct affine quantizer has (range, argmin -> 0,
argmax -> 2^b-1, reconstruction within scale/2), and by dequantization
special cases (q = 0 gives the bias exactly)."""
import numpy as np
import pytest

import oracle
from conftest import load_golden
from workloads import generic_weights




@pytest.mark.parametrize("case", [c for c in load_golden("quantize_hand.json")["cases"]
                                  if "multipliers" in c], ids=lambda c: c["name"])
def test_hand_progressions(case):
    mult = np.asarray(case["multipliers"], dtype=np.float64)
    w = (case["min"] + case["step"] * mult).astype(np.float32)
    # every value is exactly representable: the construction is exact
    assert np.all(w.astype(np.float64) == case["min"] + case["step"] * mult)
    q, s, b = oracle.quantize_affine(w[None, :], case["bits"], case["group"])
    assert q[0].tolist() == case["codes"]
    assert float(s[0, 0]) == case["scale"]
    assert float(b[0, 0]) == case["bias"]


def test_rounded_scale_decides_code():
    case = [c for c in load_golden("quantize_hand.json")["cases"]
            if c["name"].startswith("rounded fp32 scale")][0]
    w = np.asarray(case["values"], dtype=np.float32)[None, :]
    q, s, b = oracle.quantize_affine(w, case["bits"], case["group"])
    assert float(s[0, 0]) == case["scale"]
    assert float(b[0, 0]) == case["bias"]
    assert q[0].tolist() == case["codes"]


@pytest.mark.parametrize("bits", [4, 8])
def test_constant_group(bits):
    c = np.float32(0.123)
    w = np.full((3, 64), c, dtype=np.float32)
    w[1, 32:] = -2.5          # second group of row 1 constant at another value
    q, s, b = oracle.quantize_affine(w, bits, 32)
    assert np.all(q == 0)
    assert np.all(s == 0)
    assert b[0, 0] == c and b[1, 1] == np.float32(-2.5)
    wt = oracle.dequantize(q, s, b, 32)
    assert np.array_equal(wt, w.astype(np.float64))


@pytest.mark.parametrize("bits,group", [(8, 32), (8, 64), (8, 128), (4, 32), (4, 64), (4, 128)])
def test_random_group_properties(bits, group):
    w = generic_weights((11, bits, group), 37, 256, sigma=0.05)
    q, s, b = oracle.quantize_affine(w, bits, group)
    qmax = (1 << bits) - 1
    assert q.dtype == np.uint8 and q.shape == w.shape
    assert int(q.max()) <= qmax
    wg = w.reshape(37, -1, group)
    qg = q.reshape(37, -1, group)
    # argmin -> 0 and argmax -> qmax in every non-constant group
    amin = wg.argmin(axis=2)
    amax = wg.argmax(axis=2)
    assert np.all(np.take_along_axis(qg, amin[..., None], 2) == 0)
    assert np.all(np.take_along_axis(qg, amax[..., None], 2) == qmax)
    # bias is the group minimum, scale the range over qmax (to fp32 rounding)
    assert np.array_equal(b, wg.min(axis=2))
    span = wg.max(axis=2).astype(np.float64) - wg.min(axis=2)
    assert np.allclose(s, span / qmax, rtol=2 ** -23, atol=0)
    # reconstruction error at most half a step
    wt = oracle.dequantize(q, s, b, group)
    step = np.repeat(s.astype(np.float64), group, axis=1)
    assert np.all(np.abs(wt - w) <= 0.5 * step * (1 + 1e-6))


def test_dequant_endpoints():
    """q = 0 gives the bias exactly; q = 2^b - 1 gives bias + (2^b - 1) * scale."""
    codes = np.array([[0] * 32 + [255] * 32], dtype=np.uint8)
    scale = np.array([[0.375, 0.001]], dtype=np.float32)
    bias = np.array([[-1.25, 0.7]], dtype=np.float32)
    wt = oracle.dequantize(codes, scale, bias, 32)
    assert np.all(wt[0, :32] == np.float64(np.float32(-1.25)))
    expect = np.float64(np.float32(0.7)) + 255 * np.float64(np.float32(0.001))
    assert np.all(wt[0, 32:] == expect)


def test_dequant_group_indexing():
    """Each group uses its own (scale, bias): a swapped or shifted index shows."""
    codes = np.ones((2, 96), dtype=np.uint8)
    scale = np.array([[1, 2, 4], [8, 16, 32]], dtype=np.float32)
    bias = np.array([[0, 10, 20], [30, 40, 50]], dtype=np.float32)
    wt = oracle.dequantize(codes, scale, bias, 32)
    assert wt[0, 0] == 1 and wt[0, 32] == 12 and wt[0, 95] == 24
    assert wt[1, 0] == 38 and wt[1, 63] == 56 and wt[1, 64] == 82


def test_quantize_then_dequantize_roundtrip_of_codes():
    """Quantizing a dequantized grid returns the same codes (idempotence on the grid)."""
    w = generic_weights((5,), 8, 128, sigma=1.0)
    q, s, b = oracle.quantize_affine(w, 8, 64)
    wt = oracle.dequantize(q, s, b, 64).astype(np.float32)
    q2, s2, b2 = oracle.quantize_affine(wt, 8, 64)
    assert np.mean(q2 == q) > 0.99     # fp32 rounding of the grid may move a rare tie
    assert np.max(np.abs(q2.astype(int) - q.astype(int))) <= 1


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_affine(np.zeros((2, 48), np.float32), 8, 32)
    with pytest.raises(ValueError):
        oracle.quantize_affine(np.zeros((2, 64), np.float64), 8, 32)
    bad = np.zeros((1, 32), np.float32)
    bad[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_affine(bad, 8, 32)
    with pytest.raises(ValueError):
        oracle.quantize_affine(np.zeros((1, 32), np.float32), 3, 32)


def test_dense_bf16_values():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x3C23], dtype=np.uint16)
    v = oracle.dequantize_dense_bf16(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[3] == 0.0
    assert v[2] == 3.140625           # 0x4049 = 1.5703125 * 2
    assert v[4] == 0.00994873046875   # 2^-7 * (1 + 35/128)
