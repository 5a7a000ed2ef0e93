"""The scale-normalized error used to gate generated reductions
(meTile docs, "Compute-Graph Fusion" page, section "Automatic Gated
Epilogues": generated reductions are gated by a scale-normalized primitive
error).  Reading: max over all elements of |out - ref|, divided by the
largest |ref| (test infrastructure only)."""
from __future__ import annotations

import numpy as np


def scaled_error(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(out - ref)))
    if scale == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / scale
