"""Python binding of libqdm.so (the one-row quantized decode MLP for MI355X).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream.  The
names mirror the C ABI in include/qdm.h without the ``qdm_`` prefix.

The library must be built first (``python quantized_decode_mlp_amd/build.py``
or ``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqdm.so")

QDM_OK = 0
QDM_ERR_INVALID_ARG = -1
QDM_ERR_UNSUPPORTED = -2
QDM_ERR_ALIGNMENT = -3
QDM_ERR_WORKSPACE = -4
QDM_ERR_HIP = -5
QDM_ERR_TOO_LARGE = -6
NOALLOC_SCRATCH_BYTES = 16 << 20   # QDM_NOALLOC_SCRATCH_BYTES

QDM_F32, QDM_F16, QDM_BF16 = 0, 1, 2
QDM_MXFP4, QDM_MXFP8 = 0x104, 0x108       # qdm_weight.bits of the MX block-scaled formats
QDM_U4_SB16, QDM_U8_SB16 = 0x204, 0x208   # affine 4/8-bit with bf16 (scale, bias) pairs

# Every symbol include/qdm.h declares (checked by the tests).
EXPORTS = (
    "qdm_packed_q_bytes", "qdm_scale_bias_floats", "qdm_mlp_workspace_bytes",
    "qdm_gemv_gate_up_workspace_bytes", "qdm_gemv_down_workspace_bytes",
    "qdm_quantize_affine", "qdm_pack_rows", "qdm_quantize_pack_rows",
    "qdm_quantize_pack_gate_up", "qdm_pack_gate_up", "qdm_pack_dense_gate_up",
    "qdm_gemv_gate_up_swiglu", "qdm_gemv_down_residual", "qdm_gemv_linear", "qdm_mlp_decode",
    "qdm_mlp_decode_noalloc",
    "qdm_add_rmsnorm", "qdm_mlp_rmsnorm_workspace_bytes", "qdm_mlp_decode_rmsnorm",
    "qdm_mx_scale_bytes", "qdm_quantize_mx", "qdm_quantize_mx_gate_up",
    "qdm_quantize_pack_rows_sb16", "qdm_quantize_pack_gate_up_sb16",
    "qdm_status_string", "qdm_version",
)


class QdmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class qdm_weight(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("k", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("q", ctypes.c_void_p), ("scale_bias", ctypes.c_void_p),
                ("block_scales", ctypes.c_void_p)]


def _load():
    # torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch
    # first makes libqdm.so bind to that same runtime instance, so device
    # pointers and streams from torch are valid in the library's launches.
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python quantized_decode_mlp_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, sz, vp, f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    pw = ctypes.POINTER(qdm_weight)
    sig = {
        "qdm_packed_q_bytes": (sz, [i32, i32, i32]),
        "qdm_scale_bias_floats": (sz, [i32, i32, i32]),
        "qdm_mlp_workspace_bytes": (sz, [i32, ctypes.c_int, pw, pw]),
        "qdm_gemv_gate_up_workspace_bytes": (sz, [i32, ctypes.c_int, pw]),
        "qdm_gemv_down_workspace_bytes": (sz, [i32, ctypes.c_int, pw]),
        "qdm_quantize_affine": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, vp, vp]),
        "qdm_pack_rows": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "qdm_quantize_pack_rows": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, vp]),
        "qdm_quantize_pack_gate_up": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, vp, vp]),
        "qdm_pack_gate_up": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "qdm_pack_dense_gate_up": (ctypes.c_int, [vp, vp, i32, i32, vp]),
        "qdm_gemv_gate_up_swiglu": (ctypes.c_int, [vp, i32, ctypes.c_int, pw, vp, sz, vp, vp]),
        "qdm_gemv_down_residual": (ctypes.c_int, [vp, vp, i32, ctypes.c_int, pw, vp, sz, vp, vp]),
        "qdm_gemv_linear": (ctypes.c_int, [vp, i32, ctypes.c_int, ctypes.POINTER(qdm_weight), vp, vp, vp]),
        "qdm_mlp_decode": (ctypes.c_int, [vp, vp, i32, ctypes.c_int, ctypes.POINTER(qdm_weight),
                                          ctypes.POINTER(qdm_weight), vp, sz, vp, vp]),
        "qdm_mlp_decode_noalloc": (ctypes.c_int, [vp, vp, i32, ctypes.c_int, pw, pw, vp, vp]),
        "qdm_add_rmsnorm": (ctypes.c_int, [vp, vp, vp, i32, i32, f32, ctypes.c_int, vp, vp, vp]),
        "qdm_mlp_rmsnorm_workspace_bytes": (sz, [i32, ctypes.c_int, pw, pw]),
        "qdm_mlp_decode_rmsnorm": (ctypes.c_int, [vp, vp, vp, f32, i32, ctypes.c_int, ctypes.POINTER(qdm_weight),
                                                  ctypes.POINTER(qdm_weight), vp, sz, vp, vp, vp]),
        "qdm_mx_scale_bytes": (sz, [i32, i32]),
        "qdm_quantize_pack_rows_sb16": (ctypes.c_int, [vp, i32, i32, i32, i32, vp, vp]),
        "qdm_quantize_pack_gate_up_sb16": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, vp, vp]),
        "qdm_quantize_mx": (ctypes.c_int, [vp, i32, i32, i32, vp, vp]),
        "qdm_quantize_mx_gate_up": (ctypes.c_int, [vp, vp, i32, i32, i32, vp, vp]),
        "qdm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "qdm_version": (ctypes.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
LIB_PATH = _LIB_PATH


def status_string(status: int) -> str:
    return _lib.qdm_status_string(int(status)).decode()


def version() -> int:
    return int(_lib.qdm_version())


def _check(status: int, where: str) -> None:
    if status != QDM_OK:
        raise QdmError(int(status), where)


def packed_q_bytes(n: int, k: int, bits: int) -> int:
    return int(_lib.qdm_packed_q_bytes(n, k, bits))


def scale_bias_floats(n: int, k: int, group: int) -> int:
    return int(_lib.qdm_scale_bias_floats(n, k, group))


def mlp_workspace_bytes(m: int, act: int, gate_up: "Weight", down: "Weight") -> int:
    return int(_lib.qdm_mlp_workspace_bytes(m, act, ctypes.byref(gate_up.descriptor), ctypes.byref(down.descriptor)))


def mlp_rmsnorm_workspace_bytes(m: int, act: int, gate_up: "Weight", down: "Weight") -> int:
    return int(_lib.qdm_mlp_rmsnorm_workspace_bytes(m, act, ctypes.byref(gate_up.descriptor),
                                                    ctypes.byref(down.descriptor)))


def gemv_gate_up_workspace_bytes(m: int, act: int, gate_up: "Weight") -> int:
    return int(_lib.qdm_gemv_gate_up_workspace_bytes(m, act, ctypes.byref(gate_up.descriptor)))


def gemv_down_workspace_bytes(m: int, act: int, down: "Weight") -> int:
    return int(_lib.qdm_gemv_down_workspace_bytes(m, act, ctypes.byref(down.descriptor)))


# ------------------------------------------------------------------ host: quantize / pack

def _host(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_affine(w, bits: int, group: int):
    """fp32 [n, k] -> (codes uint8 [n, k], scale fp32 [n, k/g], bias fp32 [n, k/g])."""
    w = _host(w, np.float32)
    n, k = w.shape
    codes = np.empty((n, k), np.uint8)
    ng = k // group if group > 0 else 0
    scale = np.empty((n, max(ng, 1)), np.float32)
    bias = np.empty((n, max(ng, 1)), np.float32)
    _check(_lib.qdm_quantize_affine(_ptr(w), n, k, bits, group, _ptr(codes), _ptr(scale), _ptr(bias)),
           "qdm_quantize_affine")
    return codes, scale, bias


def _out_buffers(n, k, bits, group, rows_mult=1):
    qb = packed_q_bytes(n, k, bits)
    sbf = scale_bias_floats(n, k, group)
    if qb == 0 or sbf == 0:
        raise QdmError(QDM_ERR_INVALID_ARG, "packed sizes")
    return np.empty(qb * rows_mult, np.uint8), np.empty(sbf * rows_mult, np.float32)


def pack_rows(codes, scale, bias, bits: int, group: int):
    """Logical codes/scale/bias -> (packed codes uint8 [n, k*bits/8], scale_bias fp32 [n, k/g, 2])."""
    codes = _host(codes, np.uint8)
    scale = _host(scale, np.float32)
    bias = _host(bias, np.float32)
    n, k = codes.shape
    q, sb = _out_buffers(n, k, bits, group)
    _check(_lib.qdm_pack_rows(_ptr(codes), _ptr(scale), _ptr(bias), n, k, bits, group, _ptr(q), _ptr(sb)),
           "qdm_pack_rows")
    return q.reshape(n, -1), sb.reshape(n, k // group, 2)


def quantize_pack_rows(w, bits: int, group: int):
    w = _host(w, np.float32)
    n, k = w.shape
    q, sb = _out_buffers(n, k, bits, group)
    _check(_lib.qdm_quantize_pack_rows(_ptr(w), n, k, bits, group, _ptr(q), _ptr(sb)),
           "qdm_quantize_pack_rows")
    return q.reshape(n, -1), sb.reshape(n, k // group, 2)


def quantize_pack_gate_up(w_gate, w_up, bits: int, group: int):
    """-> (codes uint8 [ffn, 2, d*bits/8], scale_bias fp32 [ffn, 2, d/g, 2])."""
    wg = _host(w_gate, np.float32)
    wu = _host(w_up, np.float32)
    if wg.shape != wu.shape:
        raise ValueError("gate and up shapes differ")
    ffn, d = wg.shape
    q, sb = _out_buffers(ffn, d, bits, group, rows_mult=2)
    _check(_lib.qdm_quantize_pack_gate_up(_ptr(wg), _ptr(wu), ffn, d, bits, group, _ptr(q), _ptr(sb)),
           "qdm_quantize_pack_gate_up")
    return q.reshape(ffn, 2, -1), sb.reshape(ffn, 2, d // group, 2)


def quantize_pack_rows_sb16(w, bits: int, group: int):
    """fp32 [n, k] -> (codes uint8 [n, k*bits/8], bf16 (scale, bias) uint16 [n, k/g, 2])."""
    w = _host(w, np.float32)
    n, k = w.shape
    q = np.empty(packed_q_bytes(n, k, bits), np.uint8)
    sb = np.empty(scale_bias_floats(n, k, group), np.uint16)
    _check(_lib.qdm_quantize_pack_rows_sb16(_ptr(w), n, k, bits, group, _ptr(q), _ptr(sb)),
           "qdm_quantize_pack_rows_sb16")
    return q.reshape(n, -1), sb.reshape(n, k // group, 2)


def quantize_pack_gate_up_sb16(w_gate, w_up, bits: int, group: int):
    """-> (codes uint8 [ffn, 2, d*bits/8], bf16 pairs uint16 [ffn, 2, d/g, 2])."""
    wg, wu = _host(w_gate, np.float32), _host(w_up, np.float32)
    if wg.shape != wu.shape:
        raise ValueError("gate and up shapes differ")
    ffn, d = wg.shape
    q = np.empty(2 * packed_q_bytes(ffn, d, bits), np.uint8)
    sb = np.empty(2 * scale_bias_floats(ffn, d, group), np.uint16)
    _check(_lib.qdm_quantize_pack_gate_up_sb16(_ptr(wg), _ptr(wu), ffn, d, bits, group, _ptr(q), _ptr(sb)),
           "qdm_quantize_pack_gate_up_sb16")
    return q.reshape(ffn, 2, -1), sb.reshape(ffn, 2, d // group, 2)


def mx_scale_bytes(n: int, k: int) -> int:
    return int(_lib.qdm_mx_scale_bytes(n, k))


def _mx_buffers(n, k, fmt, rows_mult=1):
    qb, eb = packed_q_bytes(n, k, fmt), mx_scale_bytes(n, k)
    if qb == 0 or eb == 0:
        raise QdmError(QDM_ERR_INVALID_ARG, "MX sizes")
    return np.empty(qb * rows_mult, np.uint8), np.empty(eb * rows_mult, np.uint8)


def quantize_mx(w, fmt: int):
    """fp32 [n, k] -> (stored codes uint8 [n, k or k/2], E8M0 scales uint8 [n, k/32]); fmt QDM_MXFP4/8."""
    w = _host(w, np.float32)
    n, k = w.shape
    q, e = _mx_buffers(n, k, fmt)
    _check(_lib.qdm_quantize_mx(_ptr(w), n, k, fmt, _ptr(q), _ptr(e)), "qdm_quantize_mx")
    return q.reshape(n, -1), e.reshape(n, -1)


def quantize_mx_gate_up(w_gate, w_up, fmt: int):
    """-> (codes uint8 [ffn, 2, ...], E8M0 scales uint8 [ffn, 2, d/32]), rows interleaved."""
    wg, wu = _host(w_gate, np.float32), _host(w_up, np.float32)
    if wg.shape != wu.shape:
        raise ValueError("gate and up shapes differ")
    ffn, d = wg.shape
    q, e = _mx_buffers(ffn, d, fmt, rows_mult=2)
    _check(_lib.qdm_quantize_mx_gate_up(_ptr(wg), _ptr(wu), ffn, d, fmt, _ptr(q), _ptr(e)),
           "qdm_quantize_mx_gate_up")
    return q.reshape(ffn, 2, -1), e.reshape(ffn, 2, -1)


def pack_gate_up(gate_codes, gate_scale, gate_bias, up_codes, up_scale, up_bias, bits: int, group: int):
    gc, uc = _host(gate_codes, np.uint8), _host(up_codes, np.uint8)
    gs, gb = _host(gate_scale, np.float32), _host(gate_bias, np.float32)
    us, ub = _host(up_scale, np.float32), _host(up_bias, np.float32)
    ffn, d = gc.shape
    q, sb = _out_buffers(ffn, d, bits, group, rows_mult=2)
    _check(_lib.qdm_pack_gate_up(_ptr(gc), _ptr(gs), _ptr(gb), _ptr(uc), _ptr(us), _ptr(ub),
                                 ffn, d, bits, group, _ptr(q), _ptr(sb)), "qdm_pack_gate_up")
    return q.reshape(ffn, 2, -1), sb.reshape(ffn, 2, d // group, 2)


def pack_dense_gate_up(gate_bf16, up_bf16):
    """bf16 words [ffn, d] x2 -> uint16 [ffn, 2, d]."""
    g, u = _host(gate_bf16, np.uint16), _host(up_bf16, np.uint16)
    ffn, d = g.shape
    out = np.empty((ffn, 2, d), np.uint16)
    _check(_lib.qdm_pack_dense_gate_up(_ptr(g), _ptr(u), ffn, d, _ptr(out)), "qdm_pack_dense_gate_up")
    return out


# ------------------------------------------------------------------ device

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    m = {torch.float32: QDM_F32, torch.float16: QDM_F16, torch.bfloat16: QDM_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Weight:
    """A packed weight matrix resident in device memory plus its descriptor.

    For a gate/up pair, ``n`` is ffn and ``q`` holds [ffn, 2, ...] interleaved rows."""
    n: int
    k: int
    bits: int
    group: int
    q: object                       # torch uint8 (affine, MX) or int16/uint8 view (dense) on device
    scale_bias: Optional[object]    # torch float32 on device, or None for dense and MX
    block_scales: Optional[object] = None   # torch uint8 E8M0 scales on device (MX), else None
    _desc: qdm_weight = field(default=None, repr=False)

    def __post_init__(self):
        self._desc = qdm_weight(self.n, self.k, self.bits, self.group,
                                ctypes.c_void_p(self.q.data_ptr()).value,
                                None if self.scale_bias is None else
                                ctypes.c_void_p(self.scale_bias.data_ptr()).value,
                                None if self.block_scales is None else
                                ctypes.c_void_p(self.block_scales.data_ptr()).value)

    @property
    def descriptor(self) -> qdm_weight:
        return self._desc

    @staticmethod
    def from_host(n, k, bits, group, q: np.ndarray, scale_bias: Optional[np.ndarray], device="cuda",
                  block_scales: Optional[np.ndarray] = None):
        torch = _torch()
        qt = torch.from_numpy(np.ascontiguousarray(q).view(np.uint8).reshape(-1)).to(device)
        if scale_bias is None:
            sbt = None
        elif np.asarray(scale_bias).dtype == np.uint16:   # bf16 pairs: the bytes as they are
            sbt = torch.from_numpy(np.ascontiguousarray(scale_bias).view(np.uint8).reshape(-1)).to(device)
        else:
            sbt = torch.from_numpy(np.ascontiguousarray(scale_bias, dtype=np.float32).reshape(-1)).to(device)
        bst = None if block_scales is None else \
            torch.from_numpy(np.ascontiguousarray(block_scales, dtype=np.uint8).reshape(-1)).to(device)
        return Weight(n, k, bits, group, qt, sbt, bst)


def _workspace(workspace, nbytes, device):
    """(pointer, bytes) of a caller's workspace, or of a new one when none is
    given and nbytes > 0; (None, 0) when none is needed."""
    if workspace is None:
        if nbytes == 0:
            return None, 0
        workspace = _torch().empty(nbytes, dtype=_torch().uint8, device=device)
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def gemv_gate_up_swiglu(x, gate_up: Weight, h_out=None, workspace=None, stream=None):
    """x [m, d] (f32/f16/bf16, device) -> h [m, ffn] fp32."""
    torch = _torch()
    m = x.shape[0] if x.dim() == 2 else 1
    if h_out is None:
        h_out = torch.empty((m, gate_up.n), dtype=torch.float32, device=x.device)
    ws, nbytes = _workspace(workspace, gemv_gate_up_workspace_bytes(m, _dt(x), gate_up), x.device)
    _check(_lib.qdm_gemv_gate_up_swiglu(_dev(x, "x"), m, _dt(x), ctypes.byref(gate_up.descriptor), ws, nbytes,
                                        _dev(h_out, "h_out"), _stream(stream)), "qdm_gemv_gate_up_swiglu")
    return h_out


def gemv_down_residual(h, r, down: Weight, out=None, workspace=None, stream=None):
    """h [m, ffn] fp32, r [m, d] -> out [m, d] (dtype of r)."""
    torch = _torch()
    m = r.shape[0] if r.dim() == 2 else 1
    if out is None:
        out = torch.empty_like(r)
    if out.dtype != r.dtype:
        raise TypeError("out must have the dtype of r")
    ws, nbytes = _workspace(workspace, gemv_down_workspace_bytes(m, _dt(r), down), r.device)
    _check(_lib.qdm_gemv_down_residual(_dev(h, "h"), _dev(r, "r"), m, _dt(r), ctypes.byref(down.descriptor), ws,
                                       nbytes, _dev(out, "out"), _stream(stream)), "qdm_gemv_down_residual")
    return out


def gemv_linear(x, w: Weight, bias=None, out=None, stream=None):
    """A projection: out [m, n] = x [m, k] W^T (+ bias [n]), all in x's dtype."""
    torch = _torch()
    m = x.shape[0] if x.dim() == 2 else 1
    if out is None:
        out = torch.empty((m, w.n), dtype=x.dtype, device=x.device)
    if out.dtype != x.dtype or (bias is not None and bias.dtype != x.dtype):
        raise TypeError("bias and out must have the dtype of x")
    _check(_lib.qdm_gemv_linear(_dev(x, "x"), m, _dt(x), ctypes.byref(w.descriptor),
                                None if bias is None else _dev(bias, "bias"), _dev(out, "out"), _stream(stream)),
           "qdm_gemv_linear")
    return out


def mlp_decode(x, r, gate_up: Weight, down: Weight, workspace=None, out=None, stream=None):
    """The MLP: out = r + W_down (silu(W_gate x) * (W_up x)), x, r, out [m, d]."""
    torch = _torch()
    m = x.shape[0] if x.dim() == 2 else 1
    if x.dtype != r.dtype:
        raise TypeError("x and r must share a dtype")
    if out is None:
        out = torch.empty_like(r)
    if out.dtype != r.dtype:
        raise TypeError("out must have the dtype of r")
    ws, nbytes = _workspace(workspace, mlp_workspace_bytes(m, _dt(x), gate_up, down), x.device)
    _check(_lib.qdm_mlp_decode(_dev(x, "x"), _dev(r, "r"), m, _dt(x), ctypes.byref(gate_up.descriptor),
                               ctypes.byref(down.descriptor), ws, nbytes, _dev(out, "out"), _stream(stream)),
           "qdm_mlp_decode")
    return out


def mlp_decode_noalloc(x, r, gate_up: Weight, down: Weight, out=None, stream=None):
    """mlp_decode with the workspace in the library's fixed per-device array
    (NOALLOC_SCRATCH_BYTES): no allocation anywhere when ``out`` is given."""
    m = x.shape[0] if x.dim() == 2 else 1
    if x.dtype != r.dtype:
        raise TypeError("x and r must share a dtype")
    if out is None:
        out = _torch().empty_like(r)
    if out.dtype != r.dtype:
        raise TypeError("out must have the dtype of r")
    _check(_lib.qdm_mlp_decode_noalloc(_dev(x, "x"), _dev(r, "r"), m, _dt(x), ctypes.byref(gate_up.descriptor),
                                       ctypes.byref(down.descriptor), _dev(out, "out"), _stream(stream)),
           "qdm_mlp_decode_noalloc")
    return out


def add_rmsnorm(a, b, w, eps: float, s_out=None, n_out=None, stream=None):
    """s = a + b, n = rmsnorm(s) * w; returns (s, n) in the dtype of a."""
    torch = _torch()
    if not (a.dtype == b.dtype == w.dtype):
        raise TypeError("a, b and w must share a dtype")
    rows = a.shape[0] if a.dim() == 2 else 1
    n = a.shape[-1]
    s_out = torch.empty_like(a) if s_out is None else s_out
    n_out = torch.empty_like(a) if n_out is None else n_out
    _check(_lib.qdm_add_rmsnorm(_dev(a, "a"), _dev(b, "b"), _dev(w, "w"), rows, n, float(eps), _dt(a),
                                _dev(s_out, "s_out"), _dev(n_out, "n_out"), _stream(stream)),
           "qdm_add_rmsnorm")
    return s_out, n_out


def mlp_decode_rmsnorm(a, b, norm_w, eps: float, gate_up: Weight, down: Weight, workspace=None, s_out=None,
                       out=None, stream=None):
    """The decode chain: s = a + b, n = rmsnorm(s) * norm_w, out = s + MLP(n);
    a, b, out [m, d], norm_w [d], one dtype.  s goes to s_out when given."""
    torch = _torch()
    if not (a.dtype == b.dtype == norm_w.dtype):
        raise TypeError("a, b and norm_w must share a dtype")
    m = a.shape[0] if a.dim() == 2 else 1
    if out is None:
        out = torch.empty_like(a)
    if out.dtype != a.dtype or (s_out is not None and s_out.dtype != a.dtype):
        raise TypeError("out and s_out must have the dtype of a")
    ws, nbytes = _workspace(workspace, mlp_rmsnorm_workspace_bytes(m, _dt(a), gate_up, down), a.device)
    _check(_lib.qdm_mlp_decode_rmsnorm(_dev(a, "a"), _dev(b, "b"), _dev(norm_w, "norm_w"), float(eps), m, _dt(a),
                                       ctypes.byref(gate_up.descriptor), ctypes.byref(down.descriptor),
                                       ws, nbytes,
                                       None if s_out is None else _dev(s_out, "s_out"), _dev(out, "out"),
                                       _stream(stream)), "qdm_mlp_decode_rmsnorm")
    return out


__all__ = [
    "Weight", "QdmError", "qdm_weight", "EXPORTS", "LIB_PATH",
    "status_string", "version", "packed_q_bytes", "scale_bias_floats", "mlp_workspace_bytes",
    "gemv_gate_up_workspace_bytes", "gemv_down_workspace_bytes",
    "quantize_affine", "pack_rows", "quantize_pack_rows", "quantize_pack_gate_up", "pack_gate_up",
    "pack_dense_gate_up", "gemv_gate_up_swiglu", "gemv_down_residual", "gemv_linear", "mlp_decode", "add_rmsnorm",
    "mlp_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "mlp_rmsnorm_workspace_bytes", "mlp_decode_rmsnorm", "mx_scale_bytes", "quantize_mx", "quantize_mx_gate_up",
    "quantize_pack_rows_sb16", "quantize_pack_gate_up_sb16",
]
