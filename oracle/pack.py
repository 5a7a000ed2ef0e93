"""Packed byte layouts read by the GPU path, written from their definition
(test infrastructure only).

Layouts (the pages keep nibbles, scales and biases unchanged when they
repack, and offer an interleaved output-major gate/up view for one-row
decode: meTile docs, "MLX-LM Backend" page, "Dispatch Policy" section):

* 8-bit codes: one code per byte, row-major [n, k].
* 4-bit codes: two codes per byte, row-major [n, k/2]; byte i of a row holds
  code 2i in its low nibble and code 2i+1 in its high nibble.
* scale/bias: fp32 pairs, [n, k/g, 2] with (scale, bias) adjacent.
* gate/up: the two matrices' rows interleaved, [ffn, 2, ...]: packed row
  2n is gate row n and packed row 2n+1 is up row n, for codes, for the
  scale/bias pairs, and for dense bf16 weights alike.
"""
from __future__ import annotations

import numpy as np


def pack_codes(codes, bits: int) -> np.ndarray:
    """codes uint8 [n, k] (values < 2^bits) -> packed bytes [n, k*bits/8]."""
    codes = np.asarray(codes)
    if codes.ndim != 2:
        raise ValueError("codes must be 2-D")
    n, k = codes.shape
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    if bits == 8:
        return codes.astype(np.uint8).copy()
    if bits == 4:
        if k % 2:
            raise ValueError("4-bit rows need an even length")
        out = np.empty((n, k // 2), dtype=np.uint8)
        for i in range(k // 2):
            lo = codes[:, 2 * i].astype(np.uint16)
            hi = codes[:, 2 * i + 1].astype(np.uint16)
            out[:, i] = (lo + 16 * hi).astype(np.uint8)
        return out
    raise ValueError("bits must be 4 or 8")


def unpack_codes(packed, bits: int, k: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    if bits == 8:
        return packed.reshape(n, k).copy()
    if bits == 4:
        out = np.empty((n, k), dtype=np.uint8)
        out[:, 0::2] = packed % 16
        out[:, 1::2] = packed // 16
        return out
    raise ValueError("bits must be 4 or 8")


def pack_scale_bias(scale, bias) -> np.ndarray:
    """scale, bias fp32 [n, k/g] -> fp32 [n, k/g, 2]."""
    scale = np.asarray(scale, dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    if scale.shape != bias.shape:
        raise ValueError("scale and bias shapes differ")
    out = np.empty(scale.shape + (2,), dtype=np.float32)
    out[..., 0] = scale
    out[..., 1] = bias
    return out


def unpack_scale_bias(sb):
    sb = np.asarray(sb, dtype=np.float32)
    return sb[..., 0].copy(), sb[..., 1].copy()


def _interleave(gate, up):
    gate = np.asarray(gate)
    up = np.asarray(up)
    if gate.shape != up.shape:
        raise ValueError("gate and up shapes differ")
    out = np.empty((gate.shape[0], 2) + gate.shape[1:], dtype=gate.dtype)
    for n in range(gate.shape[0]):
        out[n, 0] = gate[n]
        out[n, 1] = up[n]
    return out


def pack_gate_up(gate_codes, up_codes, bits: int) -> np.ndarray:
    """-> bytes [ffn, 2, d*bits/8]: gate row n then up row n."""
    return _interleave(pack_codes(gate_codes, bits), pack_codes(up_codes, bits))


def pack_gate_up_scale_bias(gate_scale, gate_bias, up_scale, up_bias) -> np.ndarray:
    """-> fp32 [ffn, 2, d/g, 2]."""
    return _interleave(pack_scale_bias(gate_scale, gate_bias),
                       pack_scale_bias(up_scale, up_bias))


def pack_dense_gate_up(gate_bits, up_bits) -> np.ndarray:
    """bf16 bit patterns [ffn, d] x2 -> uint16 [ffn, 2, d]."""
    return _interleave(np.asarray(gate_bits, dtype=np.uint16),
                       np.asarray(up_bits, dtype=np.uint16))
