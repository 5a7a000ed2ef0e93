"""The decode MLP as its plain definition, in fp64 (test infrastructure only).

meTile docs, "Compute-Graph Fusion" page, section "Automatic Gated
Epilogues": two matmuls share the activation input, the epilogue is
silu(gate) * up, and a down projection consumes it; for one-row decode the
transformer residual is added to the down projection.  "MLX-LM Backend"
page, section "Dispatch Policy": gate and up share each activation load and
the SwiGLU epilogue precedes the only output write; the down projection's
store adds the residual (values @ weight.T + residual).

Weights enter already dequantized (fp64 [out, in]); activations as fp64
values.  Nothing is rounded: h and y are exact-as-fp64 references.
"""
from __future__ import annotations

import numpy as np


def silu(z):
    """silu(z) = z * sigmoid(z), evaluated without overflow:
    z / (1 + e^-z) for z >= 0 and z * e^z / (1 + e^z) for z < 0."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    zp = z[pos]
    out[pos] = zp / (1.0 + np.exp(-zp))
    zn = z[~pos]
    ez = np.exp(zn)
    out[~pos] = zn * ez / (1.0 + ez)
    return out


def _rows(a, width: int, name: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 1:
        a = a[None, :]
    if a.ndim != 2 or a.shape[1] != width:
        raise ValueError(f"{name} must be [m, {width}], got {a.shape}")
    return a


def gate_up_swiglu(x, w_gate, w_up):
    """x [m, d], w_gate/w_up [ffn, d] -> (g, u, h) each [m, ffn];
    g = x W_gate^T, u = x W_up^T, h = silu(g) * u."""
    w_gate = np.asarray(w_gate, dtype=np.float64)
    w_up = np.asarray(w_up, dtype=np.float64)
    if w_gate.shape != w_up.shape or w_gate.ndim != 2:
        raise ValueError("w_gate and w_up must both be [ffn, d]")
    x = _rows(x, w_gate.shape[1], "x")
    g = x @ w_gate.T
    u = x @ w_up.T
    return g, u, silu(g) * u


def down_residual(h, r, w_down):
    """h [m, ffn], r [m, d], w_down [d, ffn] -> y = r + h W_down^T, [m, d]."""
    w_down = np.asarray(w_down, dtype=np.float64)
    if w_down.ndim != 2:
        raise ValueError("w_down must be [d, ffn]")
    h = _rows(h, w_down.shape[1], "h")
    r = _rows(r, w_down.shape[0], "r")
    if h.shape[0] != r.shape[0]:
        raise ValueError("h and r row counts differ")
    return r + h @ w_down.T


def mlp_decode(x, r, w_gate, w_up, w_down):
    """The whole MLP: returns (h, y)."""
    _, _, h = gate_up_swiglu(x, w_gate, w_up)
    return h, down_residual(h, r, w_down)
