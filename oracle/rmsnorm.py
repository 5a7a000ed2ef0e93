"""Residual add + RMSNorm with both outputs, in fp64 (test infrastructure only).

meTile docs, "Compute-Graph Fusion" page, opening GraphBuilder example:
summed = values + residual; normalized = rms_norm(summed, weight, 1e-5);
both are graph outputs, so the lowering is one multi-output kernel.
"MLX-LM Backend" page, "Dispatch Policy" section: RMSNorm takes
BF16/FP16/FP32 values and weights and accumulates in FP32; the residual is
kept as a second output.

The pages print no RMSNorm formula.  Reading used (the usual one):
    n = s * w / sqrt(mean(s^2) + eps)        (eps inside the root,
                                               weight after normalization)
and the normalized input is the stored ``summed`` tensor, i.e. a + b rounded
once (nearest-even) to the storage dtype.
"""
from __future__ import annotations

import numpy as np


def _round_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (8 significant bits, exponent
    range of fp32), ties to even, via an explicit quantum."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    _, e = np.frexp(v[nz])              # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)             # below 2^-126 the spacing stops shrinking
    quantum = np.ldexp(1.0, e - 8)      # 8 significant bits
    out[nz] = np.rint(v[nz] / quantum) * quantum
    return out


def round_to_dtype(v, dtype: str) -> np.ndarray:
    """Nearest-even rounding of fp64 values to f32 / f16 / bf16, returned as fp64."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(v)
    raise ValueError(f"unknown dtype {dtype!r}")


def add_rmsnorm(a, b, w, eps: float, dtype: str):
    """a, b [rows, n], w [n] (values of the storage dtype) -> (s, n) in fp64.

    s = round_dtype(a + b) (a + b is exact in fp64 for these dtypes);
    n = s / sqrt(mean(s^2) + eps) * w, per row, unrounded."""
    a = np.atleast_2d(np.asarray(a, dtype=np.float64))
    b = np.atleast_2d(np.asarray(b, dtype=np.float64))
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    if a.shape != b.shape or a.shape[1] != w.shape[0]:
        raise ValueError("a, b must be [rows, n] and w [n]")
    s = round_to_dtype(a + b, dtype)
    ms = np.mean(s * s, axis=1, keepdims=True)
    n = s / np.sqrt(ms + eps) * w[None, :]
    return s, n
