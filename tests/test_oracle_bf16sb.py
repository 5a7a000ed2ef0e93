"""Pins for the oracle's affine format with bf16 (scale, bias) (CPU): the
stored pair is the bf16 nearest to the fp32 pair (checked against the bf16
neighbours), codes are the nearest grid points under the rounded pair
(brute force over all codes), a hand case, a constant group, and the
reconstruction bound."""
import numpy as np
import pytest

import oracle


def _bf16_neighbours(v):
    """The two bf16 values around fp32 v (its truncation and the next one up in magnitude)."""
    u = np.float32(v).view(np.uint32) & np.uint32(0xFFFF0000)
    lo = np.uint32(u).view(np.float32)
    hi = np.uint32(u + 0x10000).view(np.float32)
    return float(lo), float(hi)


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32), (8, 128)])
def test_pair_is_nearest_bf16(bits, group):
    rng = np.random.default_rng(bits + group)
    w = (rng.normal(size=(6, 4 * group)) * 0.02).astype(np.float32)
    _, s32, b32 = oracle.quantize_affine(w, bits, group)
    _, s, b = oracle.quantize_affine_bf16sb(w, bits, group)
    for ref, got in ((s32, s), (b32, b)):
        for r, g in zip(ref.ravel(), got.ravel()):
            lo, hi = _bf16_neighbours(r)
            assert g in (lo, hi)
            assert abs(g - float(r)) <= abs(float(r) - (hi if g == lo else lo))


@pytest.mark.parametrize("bits", [4, 8])
def test_codes_brute_force(bits):
    rng = np.random.default_rng(5 * bits)
    w = (rng.normal(size=(4, 64)) * 0.05).astype(np.float32)
    q, s, b = oracle.quantize_affine_bf16sb(w, bits, 32)
    qmax = (1 << bits) - 1
    for i in range(4):
        for j in range(64):
            g = j // 32
            cands = [abs(float(w[i, j]) - (s[i, g] * c + b[i, g])) for c in range(qmax + 1)]
            best = min(cands)
            assert cands[q[i, j]] <= best * (1 + 1e-12) + 1e-300


def test_hand_case():
    w = np.zeros((1, 32), np.float32)
    w[0, :4] = [-0.5, 0.0, 0.25, 0.5 + 2 ** -12]
    q, s, b = oracle.quantize_affine_bf16sb(w, 8, 32)
    # fp32 scale (1 + 2^-12) / 255 = 0x3B808889 rounds up to the bf16 0x3B810000
    # (0.003936767578125); bias -0.5 is a bf16.  Under the rounded pair the
    # maximum sits at (1 + 2^-12) / 0.003936767578125 = 254.08 -> code 254,
    # 0.0 at 127.008 -> 127, 0.25 at 190.51 -> 191
    assert b[0, 0] == -0.5
    assert s[0, 0] == float(np.uint32(0x3B810000).view(np.float32))
    assert q[0, :4].tolist() == [0, 127, 191, 254]


def test_constant_group():
    w = np.full((1, 64), 0.3, np.float32)
    q, s, b = oracle.quantize_affine_bf16sb(w, 4, 64)
    assert s[0, 0] == 0 and np.all(q == 0)
    assert b[0, 0] == oracle.round_to_dtype(np.float64(np.float32(0.3)), "bf16")


def test_reconstruction_bound():
    rng = np.random.default_rng(9)
    w = (rng.normal(size=(8, 256)) * 0.02).astype(np.float32)
    q, s, b = oracle.quantize_affine_bf16sb(w, 8, 64)
    deq = oracle.dequantize_bf16sb(q, s, b, 64)
    step = np.repeat(s, 64, axis=1)
    # inside the range, half a step; at the clamp ends, the bias/scale rounding adds at most a step
    assert np.all(np.abs(deq - w) <= step * 1.5 + 1e-12)
