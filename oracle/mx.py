"""Block-scaled MXFP4 / MXFP8 weights, in fp64 (test infrastructure only).

meTile docs, "MLX-LM Backend" page, section "Block-Scaled MLX Primitive":
MXFP4 and MXFP8 weights carry E8M0 block scales and E2M1 (MXFP4) or E4M3
(MXFP8) element values, decoded before the matrix product.

The pages name the formats and not their parameters or the quantizer.
Reading used (the OCP Microscaling formats, which these names denote):
* a block is 32 consecutive values along k (the input dim) of one row;
* E8M0 code e is the scale 2^(e - 127) (255 would be NaN; never produced);
* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6;
* E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals below
  2^-6, largest 448; exponent and mantissa all ones is NaN (never produced);
* quantizer: the block's shared exponent is floor(log2 max|v|) minus the
  element format's largest exponent (2 for E2M1, 8 for E4M3), clamped to
  [-127, 127]; every value divided by 2^shared is rounded to the nearest
  element (ties to even mantissa) and saturated at the largest element; a
  negative value keeps its sign bit even when it rounds to zero; an
  all-zero block gets the scale code 0 and zero elements.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
# (exponent bits, mantissa bits, bias, largest exponent of a normal, largest magnitude)
FORMATS = {"mxfp4": (2, 1, 1, 2, 6.0), "mxfp8": (4, 3, 7, 8, 448.0)}


def decode_element(codes, fmt: str) -> np.ndarray:
    """Element codes (uint) -> fp64 values, from the bit fields."""
    eb, mb, bias, _, _ = FORMATS[fmt]
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> (eb + mb)) & 1, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    frac = m / float(1 << mb)
    mag = np.where(e == 0, np.ldexp(frac, 1 - bias), np.ldexp(1.0 + frac, (e - bias).astype(np.int64)))
    if fmt == "mxfp8":
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode_scale(e8m0) -> np.ndarray:
    e = np.asarray(e8m0, dtype=np.int64)
    return np.ldexp(1.0, e - 127)


def _round_element(t: np.ndarray, fmt: str) -> np.ndarray:
    """|t| (fp64, >= 0) rounded to the element grid, ties to even, saturated."""
    _, mb, bias, _, vmax = FORMATS[fmt]
    emin = 1 - bias                                  # exponent of the smallest normal
    out = np.zeros_like(t)
    nz = t > 0
    _, ex = np.frexp(t[nz])                          # t = f * 2^ex, 0.5 <= f < 1
    e = np.maximum(ex - 1, emin)                     # floor(log2 t), subnormals share emin
    quantum = np.ldexp(1.0, e - mb)
    out[nz] = np.minimum(np.rint(t[nz] / quantum) * quantum, vmax)
    return out


def _encode_element(mag: np.ndarray, neg: np.ndarray, fmt: str) -> np.ndarray:
    eb, mb, bias, _, _ = FORMATS[fmt]
    emin = 1 - bias
    code = np.zeros(mag.shape, dtype=np.int64)
    nz = mag > 0
    _, ex = np.frexp(mag[nz])
    e = ex - 1
    sub = e < emin
    m_sub = np.rint(mag[nz] / np.ldexp(1.0, emin - mb)).astype(np.int64)
    m_nor = np.rint((mag[nz] / np.ldexp(1.0, e) - 1.0) * (1 << mb)).astype(np.int64)
    code[nz] = np.where(sub, m_sub, ((e + bias) << mb) | m_nor)
    return code | (neg.astype(np.int64) << (eb + mb))


def quantize_mx(w, fmt: str):
    """w [n, k] (k a multiple of 32) -> (codes uint8 [n, k], e8m0 uint8 [n, k/32])."""
    _, _, _, emax, _ = FORMATS[fmt]
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 32")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip(ex - 1 - emax, -127, 127)
    shared = np.where(amax > 0, shared, -127)
    t = np.abs(blocks) / np.ldexp(1.0, shared)[:, :, None]
    mag = _round_element(t, fmt)
    codes = _encode_element(mag, blocks < 0, fmt)
    return codes.reshape(n, k).astype(np.uint8), (shared + 127).astype(np.uint8)


def dequantize_mx(codes, e8m0, fmt: str) -> np.ndarray:
    codes = np.asarray(codes)
    n, k = codes.shape
    vals = decode_element(codes, fmt).reshape(n, k // BLOCK, BLOCK)
    return (vals * decode_scale(e8m0)[:, :, None]).reshape(n, k)


def pack_mx_codes(codes, fmt: str) -> np.ndarray:
    """Element codes [n, k] -> stored bytes: one per byte (MXFP8), or two per
    byte, code 2i in the low nibble and 2i + 1 in the high nibble (MXFP4)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "mxfp8":
        return codes.copy()
    return (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)
