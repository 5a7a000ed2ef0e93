"""The C-ABI library (CPU): it loads, exports every symbol include/qdm.h
declares, and rejects bad arguments before launching anything.

Every device-entry-point call here carries at least one invalid argument, so
validation returns before any HIP call; no compute runs without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_decode_mlp_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qdm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qdm_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    declared = _declared()
    assert set(declared) == set(q.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(qdm_[a-z0-9_]+)\b", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing


def test_gfx950_code_object_present():
    # the library's offload bundle names its target id
    data = open(q.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings_and_version():
    assert q.status_string(0) == "ok"
    assert "workspace" in q.status_string(q.QDM_ERR_WORKSPACE)
    assert q.status_string(12345) == "unknown status"
    assert q.version() >= 100


def test_sizes():
    assert q.packed_q_bytes(4096, 12288, 8) == 4096 * 12288
    assert q.packed_q_bytes(4096, 14336, 4) == 4096 * 14336 // 2
    assert q.packed_q_bytes(1536, 8960, 16) == 1536 * 8960 * 2
    assert q.packed_q_bytes(0, 10, 8) == 0 and q.packed_q_bytes(2, 3, 4) == 0
    assert q.scale_bias_floats(4096, 12288, 128) == 2 * 4096 * 96
    assert q.scale_bias_floats(4, 100, 32) == 0



def _ws(fn, m, act, *ws):
    return getattr(L, fn)(m, act, *(ctypes.byref(w) for w in ws))


def test_workspace_sizes():
    """The workspace queries, from the shapes alone (no device): h, plus the
    split-K partials of the largest split a call makes."""
    bf16 = q.QDM_BF16
    # one row (Qwen3-8B-shaped uint8 g128): h only, no partials
    gu, dn = _w(n=12288, k=4096, bits=8, group=128), _w(n=4096, k=12288, bits=8, group=128)
    assert _ws("qdm_mlp_workspace_bytes", 1, bf16, gu, dn) == 12288 * 4
    assert _ws("qdm_gemv_gate_up_workspace_bytes", 1, bf16, gu) == 0
    assert _ws("qdm_gemv_down_workspace_bytes", 1, bf16, dn) == 0
    assert _ws("qdm_mlp_workspace_bytes", 3, bf16, _w(n=10, k=64), _w(n=64, k=10 * 32)) == 0   # k mismatch
    assert _ws("qdm_mlp_workspace_bytes", 1, bf16, _w(n=32, k=64), _w(n=64, k=32)) == 256   # 128 B of h, rounded
    assert _ws("qdm_mlp_workspace_bytes", 3, bf16, _w(n=64, k=64), _w(n=64, k=64)) == 768
    assert _ws("qdm_mlp_workspace_bytes", 0, bf16, gu, dn) == 0
    assert _ws("qdm_mlp_workspace_bytes", 1, 9, gu, dn) == 0
    # Llama-3-8B-shaped 4-bit g64 at 16 rows: down splits K = 14336 into 14
    # slices of 1024 on the matrix cores, fp32 partials [14][16][4096]
    gu, dn = _w(n=14336, k=4096, bits=4, group=64), _w(n=4096, k=14336, bits=4, group=64)
    part16 = 14 * 16 * 4096 * 4
    assert _ws("qdm_gemv_down_workspace_bytes", 16, bf16, dn) == part16
    assert _ws("qdm_gemv_gate_up_workspace_bytes", 16, bf16, gu) == 0
    assert _ws("qdm_mlp_workspace_bytes", 16, bf16, gu, dn) == 16 * 14336 * 4 + part16
    # fp32 rows never take the matrix-core down kernel: no partials
    assert _ws("qdm_gemv_down_workspace_bytes", 16, q.QDM_F32, dn) == 0
    # 40 rows in passes of 16 when the tiled kernels do not take the shape:
    # dense bf16 has no partials at all
    gd, dd = _w(n=8960, k=1536, bits=16, group=0), _w(n=1536, k=8960, bits=16, group=0)
    assert _ws("qdm_mlp_workspace_bytes", 40, bf16, gd, dd) == 40 * 8960 * 4
    # more than 16 rows on the tiled kernels (64 rows x 64 gate/up pairs, or
    # 64 rows x 128 outputs, per block); K is split while the tiles give fewer
    # than two blocks per CU of the 256-CU chip: at 128 rows gate/up has 448
    # tiles -> 2 slices, down 64 tiles -> 8 slices; at 2048 rows neither splits
    gu_part = 2 * 128 * 14336 * 2 * 4
    dn_part = 8 * 128 * 4096 * 4
    assert _ws("qdm_gemv_gate_up_workspace_bytes", 128, bf16, gu) == gu_part
    assert _ws("qdm_gemv_down_workspace_bytes", 128, bf16, dn) == dn_part
    assert _ws("qdm_mlp_workspace_bytes", 128, bf16, gu, dn) == 128 * 14336 * 4 + max(gu_part, dn_part)
    assert _ws("qdm_gemv_gate_up_workspace_bytes", 2048, bf16, gu) == 0
    assert _ws("qdm_gemv_down_workspace_bytes", 2048, bf16, dn) == 0
    # the chain adds two [m][d] rows of the act dtype
    assert _ws("qdm_mlp_rmsnorm_workspace_bytes", 16, bf16, gu, dn) == 16 * 14336 * 4 + 2 * 16 * 4096 * 2 + part16


def _prefill_slices(n, k, m, gate_up, kbk):
    """The tiled kernels' split rule restated: slices double while the output
    tiles times the slices give fewer than two blocks per CU (256 CUs), each
    slice keeping at least two k-blocks, at most 16."""
    bn = 64 if gate_up else 128
    tiles = -(-n // bn) * -(-m // 64)
    s = 1
    while tiles * s < 2 * 256 and 4 * s <= k // kbk and s < 16:
        s *= 2
    return s


@pytest.mark.parametrize("m", [17, 33, 64, 100, 128, 200, 256, 512, 1000, 4096])
@pytest.mark.parametrize("shape", [(14336, 4096, 4, 64), (8192, 2048, 8, 64), (12288, 4096, 8, 128),
                                   (512, 256, 8, 32), (2048, 1024, 4, 32)])
def test_workspace_covers_the_largest_split(m, shape):
    """For every row count on the tiled kernels, the queries cover the
    partials of the split the rule above picks (the launch caps the CU count
    at 256, so no device splits finer)."""
    ffn, d, bits, group = shape
    gu, dn = _w(n=ffn, k=d, bits=bits, group=group), _w(n=d, k=ffn, bits=bits, group=group)
    kbk = 128 if bits == 4 or group == 32 else 64
    sg = _prefill_slices(ffn, d, m, True, kbk)
    sd = _prefill_slices(d, ffn, m, False, kbk)
    need_gu = 0 if sg == 1 else sg * m * ffn * 2 * 4
    need_dn = 0 if sd == 1 else sd * m * d * 4
    assert _ws("qdm_gemv_gate_up_workspace_bytes", m, q.QDM_BF16, gu) >= need_gu
    assert _ws("qdm_gemv_down_workspace_bytes", m, q.QDM_BF16, dn) >= need_dn
    total = _ws("qdm_mlp_workspace_bytes", m, q.QDM_BF16, gu, dn)
    assert total >= m * ffn * 4 + max(need_gu, need_dn)


L = q._lib
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced
ODD = ctypes.c_void_p(0x10004)           # misaligned for 16-byte checks


def _w(n=64, k=256, bits=8, group=32, qp=FAKE, sb=FAKE):
    return q.qdm_weight(n, k, bits, group, qp.value if qp else None, sb.value if sb else None)


def _gu(x=FAKE, m=1, act=q.QDM_BF16, w=None, h=ctypes.c_void_p(0x20000)):
    w = _w() if w is None else w
    return L.qdm_gemv_gate_up_swiglu(x, m, act, ctypes.byref(w), None, 0, h, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), q.QDM_ERR_INVALID_ARG),
    (dict(h=None), q.QDM_ERR_INVALID_ARG),
    (dict(m=0), q.QDM_ERR_INVALID_ARG),
    (dict(m=4097), q.QDM_ERR_UNSUPPORTED),
    (dict(act=7), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(group=16)), q.QDM_ERR_UNSUPPORTED),
    (dict(w=_w(k=96, group=64)), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(bits=3)), q.QDM_ERR_UNSUPPORTED),
    (dict(w=_w(bits=16, group=32)), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(bits=16, group=0, k=100)), q.QDM_ERR_UNSUPPORTED),
    (dict(w=_w(sb=None)), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(qp=None)), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(n=0)), q.QDM_ERR_INVALID_ARG),
    (dict(w=_w(qp=ODD)), q.QDM_ERR_ALIGNMENT),
    (dict(w=_w(sb=ctypes.c_void_p(0x10002))), q.QDM_ERR_ALIGNMENT),
    (dict(x=ctypes.c_void_p(0x30004)), q.QDM_ERR_ALIGNMENT),
    (dict(h=ctypes.c_void_p(0x20004)), q.QDM_ERR_ALIGNMENT),
    (dict(h=ctypes.c_void_p(0x10000 + 256)), q.QDM_ERR_INVALID_ARG),   # h_out overlaps x ([1][256] bf16)
])
def test_gate_up_rejects(kw, expect):
    assert _gu(**kw) == expect


def test_gate_up_workspace_rejects():
    """More than 16 rows on the tiled kernels split K into the workspace."""
    w = _w(n=14336, k=4096, bits=4, group=64)
    X, H, WS = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x8000000), ctypes.c_void_p(0x20000000)
    need = L.qdm_gemv_gate_up_workspace_bytes(128, q.QDM_BF16, ctypes.byref(w))
    assert need > 0

    def f(ws=WS, wsb=need, x=X, h=H):
        return L.qdm_gemv_gate_up_swiglu(x, 128, q.QDM_BF16, ctypes.byref(w), ws, wsb, h, None)

    assert f(ws=None) == q.QDM_ERR_WORKSPACE
    assert f(wsb=need - 1) == q.QDM_ERR_WORKSPACE
    assert f(ws=ctypes.c_void_p(0x8000000 - 256)) == q.QDM_ERR_INVALID_ARG   # workspace runs into h
    assert f(ws=ctypes.c_void_p(0x100000 - 512)) == q.QDM_ERR_INVALID_ARG    # workspace runs into x
    assert f(ws=ctypes.c_void_p(0x20000008)) == q.QDM_ERR_ALIGNMENT


def test_down_rejects():
    w = _w(n=256, k=512)
    f = lambda h=FAKE, r=FAKE, m=1, act=q.QDM_F32, wt=w, out=ctypes.c_void_p(0x20000): \
        L.qdm_gemv_down_residual(h, r, m, act, ctypes.byref(wt), None, 0, out, None)
    assert f(h=None) == q.QDM_ERR_INVALID_ARG
    assert f(r=None) == q.QDM_ERR_INVALID_ARG
    assert f(out=FAKE) == q.QDM_ERR_INVALID_ARG            # out aliases h
    assert f(out=ctypes.c_void_p(0x10000 + 2048 - 16)) == q.QDM_ERR_INVALID_ARG   # out overlaps h's tail
    assert f(m=-1) == q.QDM_ERR_INVALID_ARG
    assert f(r=ODD) == q.QDM_ERR_ALIGNMENT
    assert f(wt=_w(n=256, k=500, group=32)) == q.QDM_ERR_INVALID_ARG


def test_down_workspace_rejects():
    """2..16 rows with 16-bit outputs split K on the matrix cores into the workspace."""
    w = _w(n=4096, k=14336, bits=4, group=64)
    H, R, OUT, WS = (ctypes.c_void_p(0x1000000 * i) for i in range(1, 5))
    need = L.qdm_gemv_down_workspace_bytes(16, q.QDM_BF16, ctypes.byref(w))
    assert need == 14 * 16 * 4096 * 4

    def f(ws=WS, wsb=need, r=R, out=OUT, act=q.QDM_BF16):
        return L.qdm_gemv_down_residual(H, r, 16, act, ctypes.byref(w), ws, wsb, out, None)

    assert f(ws=None) == q.QDM_ERR_WORKSPACE
    assert f(wsb=need - 256) == q.QDM_ERR_WORKSPACE
    assert f(r=ctypes.c_void_p(0x4000000 + need - 16)) == q.QDM_ERR_INVALID_ARG    # r inside the workspace
    assert f(out=ctypes.c_void_p(0x4000000 - 16)) == q.QDM_ERR_INVALID_ARG         # out runs into it
    # fp32 outputs stay on the vector kernel: nothing to split, no workspace needed
    assert L.qdm_gemv_down_workspace_bytes(16, q.QDM_F32, ctypes.byref(w)) == 0


def test_mlp_rejects():
    gu = _w(n=512, k=256)
    dn = _w(n=256, k=512)
    ws = ctypes.c_void_p(0x30000)
    out = ctypes.c_void_p(0x40000)

    def f(m=1, gu=gu, dn=dn, ws=ws, wsb=512 * 4, out=out, x=FAKE, r=ctypes.c_void_p(0x50000)):
        return L.qdm_mlp_decode(x, r, m, q.QDM_F32, ctypes.byref(gu), ctypes.byref(dn), ws, wsb, out, None)

    assert f(wsb=512 * 4 - 1) == q.QDM_ERR_WORKSPACE
    assert f(ws=None) == q.QDM_ERR_WORKSPACE
    assert f(m=2, wsb=512 * 4) == q.QDM_ERR_WORKSPACE
    assert f(dn=_w(n=256, k=1024)) == q.QDM_ERR_INVALID_ARG          # ffn mismatch
    assert f(dn=_w(n=128, k=512)) == q.QDM_ERR_INVALID_ARG           # d mismatch
    assert f(dn=_w(n=256, k=512, bits=4)) == q.QDM_ERR_UNSUPPORTED   # mixed formats
    assert f(out=ws) == q.QDM_ERR_INVALID_ARG
    # the workspace may overlap none of x, r, out (each [1][256] fp32 = 1 KiB)
    assert f(x=ctypes.c_void_p(0x30000 + 512 * 4 - 16)) == q.QDM_ERR_INVALID_ARG
    assert f(r=ctypes.c_void_p(0x30000 - 1024 + 16)) == q.QDM_ERR_INVALID_ARG
    assert f(out=ctypes.c_void_p(0x30000 + 1024)) == q.QDM_ERR_INVALID_ARG
    assert f(x=None) == q.QDM_ERR_INVALID_ARG
    assert f(out=ODD) == q.QDM_ERR_ALIGNMENT


def test_mx_weight_rejects():
    """MX descriptors: group 32 and block scales required; only one row on the
    streaming kernel (several rows are rejected before anything runs)."""
    X, OUT = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)

    def mxw(n=256, k=512, bits=q.QDM_MXFP8, group=32, bs=FAKE):
        return q.qdm_weight(n, k, bits, group, FAKE.value, None, bs.value if bs else None)

    def lin(w, m=1):
        return L.qdm_gemv_linear(X, m, q.QDM_BF16, ctypes.byref(w), None, OUT, None)

    assert lin(mxw(group=64)) == q.QDM_ERR_UNSUPPORTED
    assert lin(mxw(bs=None)) == q.QDM_ERR_INVALID_ARG
    assert lin(mxw(k=500)) == q.QDM_ERR_INVALID_ARG
    assert lin(mxw(), m=2) == q.QDM_ERR_UNSUPPORTED
    assert lin(mxw(k=65536)) == q.QDM_ERR_UNSUPPORTED                # x does not fit the LDS stage
    assert lin(mxw(bits=q.QDM_MXFP4), m=16) == q.QDM_ERR_UNSUPPORTED


def test_linear_rejects():
    X, BIAS, OUT = (ctypes.c_void_p(0x10000 * i) for i in range(1, 4))

    def f(x=X, m=1, dt=q.QDM_BF16, w=None, bias=BIAS, out=OUT):
        w = _w(n=300, k=256) if w is None else w
        return L.qdm_gemv_linear(x, m, dt, ctypes.byref(w), bias, out, None)

    assert f(x=None) == q.QDM_ERR_INVALID_ARG
    assert f(out=None) == q.QDM_ERR_INVALID_ARG
    assert f(out=X) == q.QDM_ERR_INVALID_ARG                          # out aliases x
    assert f(out=BIAS) == q.QDM_ERR_INVALID_ARG                       # out aliases bias
    assert f(m=0) == q.QDM_ERR_INVALID_ARG
    assert f(m=4097) == q.QDM_ERR_UNSUPPORTED
    assert f(dt=5) == q.QDM_ERR_INVALID_ARG
    assert f(w=_w(n=300, k=256, bits=2)) == q.QDM_ERR_UNSUPPORTED
    assert f(w=_w(n=300, k=250, group=32)) == q.QDM_ERR_INVALID_ARG
    assert f(bias=ODD) == q.QDM_ERR_ALIGNMENT
    assert f(x=ODD) == q.QDM_ERR_ALIGNMENT


def test_chain_rejects():
    gu = _w(n=512, k=256)
    dn = _w(n=256, k=512)
    A, B, NW, S, OUT, WS = (ctypes.c_void_p(0x10000 * i) for i in range(1, 7))
    need = _ws("qdm_mlp_rmsnorm_workspace_bytes", 1, q.QDM_BF16, gu, dn)
    assert need == 512 * 4 + 2 * 512
    assert _ws("qdm_mlp_rmsnorm_workspace_bytes", 3, q.QDM_F32, gu, dn) == 3 * 512 * 4 + 2 * 3 * 256 * 4
    assert _ws("qdm_mlp_rmsnorm_workspace_bytes", 0, q.QDM_F32, gu, dn) == 0

    def f(a=A, b=B, nw=NW, eps=1e-5, m=1, dt=q.QDM_BF16, gu=gu, dn=dn, ws=WS, wsb=need, s=S, out=OUT):
        return L.qdm_mlp_decode_rmsnorm(a, b, nw, eps, m, dt, ctypes.byref(gu), ctypes.byref(dn), ws, wsb, s,
                                        out, None)

    assert f(wsb=need - 1) == q.QDM_ERR_WORKSPACE
    assert f(ws=None) == q.QDM_ERR_WORKSPACE
    assert f(m=2) == q.QDM_ERR_WORKSPACE
    assert f(nw=None) == q.QDM_ERR_INVALID_ARG
    assert f(out=None) == q.QDM_ERR_INVALID_ARG
    assert f(s=OUT) == q.QDM_ERR_INVALID_ARG                          # s_out aliases out
    assert f(ws=A, wsb=need) == q.QDM_ERR_INVALID_ARG                 # workspace aliases a
    assert f(nw=ctypes.c_void_p(0x60000 + 256)) == q.QDM_ERR_INVALID_ARG   # norm weight inside the workspace
    assert f(eps=float("nan")) == q.QDM_ERR_INVALID_ARG
    assert f(eps=-1.0) == q.QDM_ERR_INVALID_ARG
    assert f(dt=7) == q.QDM_ERR_INVALID_ARG
    assert f(m=4097) == q.QDM_ERR_UNSUPPORTED
    assert f(dn=_w(n=256, k=1024)) == q.QDM_ERR_INVALID_ARG          # ffn mismatch
    assert f(dn=_w(n=256, k=512, bits=4)) == q.QDM_ERR_UNSUPPORTED   # mixed formats
    assert f(b=ODD) == q.QDM_ERR_ALIGNMENT
    assert f(s=ODD) == q.QDM_ERR_ALIGNMENT


def test_rmsnorm_rejects():
    A, B, W, S, N = (ctypes.c_void_p(0x10000 * i) for i in range(1, 6))

    def f(a=A, b=B, w=W, rows=1, n=256, eps=1e-5, dt=q.QDM_F16, s=S, nn=N):
        return L.qdm_add_rmsnorm(a, b, w, rows, n, eps, dt, s, nn, None)

    assert f(a=None) == q.QDM_ERR_INVALID_ARG
    assert f(rows=0) == q.QDM_ERR_INVALID_ARG
    assert f(n=-3) == q.QDM_ERR_INVALID_ARG
    assert f(eps=float("nan")) == q.QDM_ERR_INVALID_ARG
    assert f(eps=-1.0) == q.QDM_ERR_INVALID_ARG
    assert f(dt=5) == q.QDM_ERR_INVALID_ARG
    assert f(nn=S) == q.QDM_ERR_INVALID_ARG
    assert f(nn=A) == q.QDM_ERR_INVALID_ARG
    assert f(w=ODD) == q.QDM_ERR_ALIGNMENT


def test_host_pack_rejects():
    import numpy as np
    w = np.zeros((4, 64), np.float32)
    with pytest.raises(q.QdmError) as e:
        q.quantize_affine(w, 8, 48)
    assert e.value.status == q.QDM_ERR_UNSUPPORTED
    w[1, 2] = np.nan
    with pytest.raises(q.QdmError) as e:
        q.quantize_pack_rows(w, 8, 32)
    assert e.value.status == q.QDM_ERR_INVALID_ARG
    codes = np.full((2, 32), 16, np.uint8)
    s = np.zeros((2, 1), np.float32)
    with pytest.raises(q.QdmError):
        q.pack_rows(codes, s, s, 4, 32)


def test_one_hip_runtime_in_process():
    """libqdm.so binds to the HIP runtime torch loaded, so torch's device
    pointers and streams are valid in its launches (two runtimes would not
    share them)."""
    paths = {l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l}
    assert len(paths) == 1, paths
