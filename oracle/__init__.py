"""fp64 CPU oracle for the one-row affine-quantized decode MLP.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product (the C-ABI library and its Python binding) never does, and this
package imports nothing from the product: the two share no code.

What it computes (plain definitions, numpy, float64):

* ``quantize_affine`` / ``dequantize`` -- affine group quantization along the
  input dim, groups of 32/64/128 (meTile docs, "MLX-LM Backend" page, the
  affine INT8 / 4-bit passages: per-group scales and biases, nibbles).
* ``quantize_affine_bf16sb`` / ``dequantize_bf16sb`` -- the same format with
  bf16 (scale, bias) pairs.
* ``pack_*`` / ``unpack_*`` -- the packed byte layouts the GPU path reads.
* ``gate_up_swiglu`` -- h = silu(W_gate x) * (W_up x) ("Compute-Graph Fusion"
  page, section "Automatic Gated Epilogues").
* ``down_residual`` -- y = r + W_down h (same section, residual epilogue;
  "MLX-LM Backend" page, section "Dispatch Policy", typed residual store).
* ``add_rmsnorm`` -- s = a + b, n = rms_norm(s, w, eps), both returned
  ("Compute-Graph Fusion" page, opening GraphBuilder example).
* ``mlp_decode_rmsnorm`` -- the decode chain: add + RMSNorm feeding the MLP,
  the sum as its residual ("Compute-Graph Fusion" page, GraphBuilder example
  and "Automatic Gated Epilogues").
* ``linear`` -- y = x W^T + b, the one-row vocabulary and attention
  projections ("MLX-LM Backend" page, the passages on vocabulary and
  attention-projection compression).
* ``quantize_mx`` / ``dequantize_mx`` / ``decode_element`` / ``pack_mx_codes``
  -- MXFP4 / MXFP8 block-scaled weights ("MLX-LM Backend" page, section
  "Block-Scaled MLX Primitive"; read as the OCP Microscaling formats).
* ``scaled_error`` -- max|out - ref| / max|ref|, the scale-normalized error
  ("Compute-Graph Fusion" page, section "Automatic Gated Epilogues").

Pins: every function is checked by ``tests/test_oracle_*.py`` against closed
forms, textbook values, hand-derived fixtures under ``tests/golden/`` and a
brute-force rational implementation on tiny inputs.  No function here is
"parity unpinned".
"""
from .quantize import (quantize_affine, dequantize, dequantize_dense_bf16, quantize_affine_bf16sb,
                       dequantize_bf16sb)
from .pack import (pack_codes, unpack_codes, pack_scale_bias, unpack_scale_bias,
                   pack_gate_up, pack_gate_up_scale_bias, pack_dense_gate_up)
from .mlp import silu, gate_up_swiglu, down_residual, mlp_decode
from .rmsnorm import round_to_dtype, add_rmsnorm
from .chain import mlp_decode_rmsnorm
from .linear import linear
from .mx import quantize_mx, dequantize_mx, decode_element, decode_scale, pack_mx_codes
from .compare import scaled_error

__all__ = [
    "quantize_affine", "dequantize", "dequantize_dense_bf16", "quantize_affine_bf16sb", "dequantize_bf16sb",
    "pack_codes", "unpack_codes", "pack_scale_bias", "unpack_scale_bias",
    "pack_gate_up", "pack_gate_up_scale_bias", "pack_dense_gate_up",
    "silu", "gate_up_swiglu", "down_residual", "mlp_decode",
    "round_to_dtype", "add_rmsnorm", "mlp_decode_rmsnorm", "linear", "scaled_error",
    "quantize_mx", "dequantize_mx", "decode_element", "decode_scale", "pack_mx_codes",
]
