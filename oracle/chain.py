"""The decode chain across the layer boundary, in fp64 (test infrastructure only).

meTile docs, "Compute-Graph Fusion" page: the opening GraphBuilder example
adds a residual and applies RMSNorm, keeping the sum as an output; section
"Automatic Gated Epilogues" gives the gated MLP whose one-row down
projection adds the transformer residual.  Chained, the normalized row is
the MLP's input and the sum is its residual.

Reading used (the pages do not write the chain out): the normalized row is a
tensor of the storage dtype between the two ops, so it is rounded once to
that dtype before the MLP; the residual is the stored sum s.  Nothing after
that is rounded.
"""
from __future__ import annotations

from .mlp import mlp_decode
from .rmsnorm import add_rmsnorm, round_to_dtype


def mlp_decode_rmsnorm(a, b, norm_w, eps: float, dtype: str, w_gate, w_up, w_down):
    """a, b [m, d], norm_w [d] (values of `dtype`), dequantized fp64 weights
    -> (s, x, h, y): s = round(a + b), x = round(rmsnorm(s) * norm_w),
    h = silu(W_gate x) * (W_up x), y = s + W_down h."""
    s, n = add_rmsnorm(a, b, norm_w, eps, dtype)
    x = round_to_dtype(n, dtype)
    h, y = mlp_decode(x, s, w_gate, w_up, w_down)
    return s, x, h, y
