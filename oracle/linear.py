"""A one-row decode projection, in fp64 (test infrastructure only).

meTile docs, "MLX-LM Backend" page, the passages on vocabulary compression
(an untied lm_head, or a tied embedding table used as the linear output map,
patched for one-row decode only) and on attention-projection compression
(q_proj, k_proj, v_proj, o_proj with their projection biases preserved):
each is the linear map y = x W^T + b on the one-row activation.

Weights enter already dequantized (fp64 [n, k]); nothing is rounded.
"""
from __future__ import annotations

import numpy as np


def linear(x, w, bias=None):
    """x [m, k], w [n, k], bias [n] or None -> y = x W^T (+ bias), [m, n]."""
    w = np.asarray(w, dtype=np.float64)
    if w.ndim != 2:
        raise ValueError("w must be [n, k]")
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    if x.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"x must be [m, {w.shape[1]}], got {x.shape}")
    y = x @ w.T
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64).reshape(-1)
        if b.shape[0] != w.shape[0]:
            raise ValueError("bias must be [n]")
        y = y + b[None, :]
    return y
