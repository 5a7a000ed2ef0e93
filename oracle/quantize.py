"""Affine group quantization, written out step by step (test infrastructure only).

Source: meTile docs, "MLX-LM Backend" page.  The affine INT8 format keeps a
scale and a bias per group (intro and "Dispatch Policy" sections); group
sizes 32, 64 and 128 run along the input dimension; the 4-bit repack keeps
"nibbles, scales, and biases" without requantizing ("Dispatch Policy").
The pages print no quantizer formula.  The reading used here (the plainest
one consistent with "scale" and "bias" and with w = scale*q + bias):

    per row n and group j (columns [j*g, (j+1)*g)):
        mn, mx  = min, max of the fp32 weights          (exact)
        scale   = fp32( (fp64(mx) - fp64(mn)) / (2^bits - 1) )   nearest-even
        bias    = mn      (a zero minimum is stored as +0)
        q       = clamp( rint( (fp64(w) - fp64(bias)) / fp64(scale) ), 0, 2^bits-1 )
    if the fp32 scale is 0 (mx == mn, or the range underflows): all q = 0.

Every step is one IEEE fp64 operation in a fixed order, so the result is
unique: an independent implementation must reproduce it bit for bit.
Dequantization is w~ = fp64(scale) * q + fp64(bias).
"""
from __future__ import annotations

import numpy as np


def _check_group(k: int, group: int) -> None:
    if group <= 0 or k % group != 0:
        raise ValueError(f"input dim {k} is not a multiple of group {group}")


def quantize_affine(w, bits: int, group: int):
    """Quantize fp32 ``w`` [n, k] -> (codes uint8 [n, k], scale fp32 [n, k/g], bias fp32 [n, k/g])."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise ValueError("w must be a 2-D float32 array")
    if not np.all(np.isfinite(w)):
        raise ValueError("w must be finite")
    n, k = w.shape
    _check_group(k, group)
    qmax = (1 << bits) - 1
    wg = w.reshape(n, k // group, group)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    span = mx.astype(np.float64) - mn.astype(np.float64)
    scale = (span / np.float64(qmax)).astype(np.float32)
    bias = mn.copy()
    bias[bias == 0] = np.float32(0.0)       # -0 and +0 minima are stored alike
    live = scale != 0
    denom = np.where(live, scale.astype(np.float64), 1.0)[..., None]
    t = (wg.astype(np.float64) - bias.astype(np.float64)[..., None]) / denom
    q = np.clip(np.rint(t), 0, qmax)
    q = np.where(live[..., None], q, 0.0)
    return q.astype(np.uint8).reshape(n, k), scale, bias


def dequantize(codes, scale, bias, group: int) -> np.ndarray:
    """w~[n, k] = fp64(scale[n, k//g]) * q[n, k] + fp64(bias[n, k//g]), in fp64."""
    codes = np.asarray(codes)
    n, k = codes.shape
    _check_group(k, group)
    s = np.repeat(np.asarray(scale, dtype=np.float32).astype(np.float64), group, axis=1)
    b = np.repeat(np.asarray(bias, dtype=np.float32).astype(np.float64), group, axis=1)
    if s.shape != (n, k) or b.shape != (n, k):
        raise ValueError("scale/bias shape does not match codes and group")
    return s * codes.astype(np.float64) + b


def dequantize_dense_bf16(bits) -> np.ndarray:
    """Dense bf16 weights (uint16 bit patterns) -> their exact values in fp64.

    A bf16 value is the upper half of the fp32 with the same bits; the lower
    16 fraction bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def quantize_affine_bf16sb(w, bits: int, group: int):
    """The same affine format with its (scale, bias) stored as bf16 -- the
    dtype MLX keeps them in for bf16 models ("MLX-LM Backend": affine
    weights keep per-group scales and biases; their storage type is not
    printed).  Reading used: scale and bias as in ``quantize_affine``, each
    rounded once to bf16 (nearest-even), then every code chosen against the
    rounded pair, q = clamp(rint((fp64(w) - fp64(bias_bf16)) / fp64(scale_bf16)),
    0, 2^bits - 1) (all 0 when the rounded scale is 0), so that dequantization
    with the stored pair is what the codes were chosen for.
    Returns (codes uint8 [n, k], scale [n, k/g], bias [n, k/g]) with the
    bf16 values in fp64."""
    from .rmsnorm import round_to_dtype
    _, scale32, bias32 = quantize_affine(w, bits, group)
    n, k = np.asarray(w).shape
    qmax = (1 << bits) - 1
    scale = round_to_dtype(scale32.astype(np.float64), "bf16")
    bias = round_to_dtype(bias32.astype(np.float64), "bf16")
    live = scale != 0
    wg = np.asarray(w, dtype=np.float32).reshape(n, k // group, group).astype(np.float64)
    denom = np.where(live, scale, 1.0)[..., None]
    q = np.clip(np.rint((wg - bias[..., None]) / denom), 0, qmax)
    q = np.where(live[..., None], q, 0.0)
    return q.astype(np.uint8).reshape(n, k), scale, bias


def dequantize_bf16sb(codes, scale, bias, group: int) -> np.ndarray:
    """w~ = scale * q + bias with the bf16 pair (given as fp64 values)."""
    codes = np.asarray(codes)
    s = np.repeat(np.asarray(scale, dtype=np.float64), group, axis=1)
    b = np.repeat(np.asarray(bias, dtype=np.float64), group, axis=1)
    return s * codes.astype(np.float64) + b
