"""GPU parity with more than 16 rows through the C ABI: the tiled prefill
kernels (64 rows x 64 outputs per block; 8/4-bit affine with either pair
storage and MX weights, 16-bit activations) and, for the other formats,
passes of 16 rows through the few-row kernels.

Bars as for the MLP: h within 1e-5 scaled error, y within 5e-3 (bf16) of the
fp64 oracle; the chain bitwise equal to add + RMSNorm then the MLP."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import H_TOL, TOL, from_device, generic_case, to_device, workload_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU")
    import quantized_decode_mlp_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


def _qdm():
    import quantized_decode_mlp_amd as qdm
    return qdm


def _check(ow, pw, x, r, act):
    qdm = _qdm()
    gu, dn = pw
    xd, rd = to_device(x), to_device(r)
    h = qdm.gemv_gate_up_swiglu(xd, gu)
    y = qdm.mlp_decode(xd, rd, gu, dn)
    torch.cuda.synchronize()
    h_ref, y_ref = oracle.mlp_decode(x.values, r.values, ow.wg, ow.wu, ow.wd)
    eh = oracle.scaled_error(from_device(h), h_ref)
    ey = oracle.scaled_error(from_device(y), y_ref)
    print(f"  h err {eh:.3e}  y err {ey:.3e}", flush=True)
    assert eh <= H_TOL, eh
    assert ey <= TOL[act], ey


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("bits,group", [(8, 32), (8, 64), (8, 128), (4, 32), (4, 64), (4, 128)])
@pytest.mark.parametrize("m", [17, 64, 130])
def test_prefill_rows(m, bits, group, act):
    """Ragged row tiles (17, 130), one full tile (64); every group width."""
    print(f"[prefill] m={m} bits={bits} group={group} act={act}", flush=True)
    d, ffn = 1024, 1536
    ow, pw = generic_case((m, bits, group, 7), d, ffn, bits, group)
    x = W.generic_act((m, 1), (m, d), act)
    r = W.generic_act((m, 2), (m, d), act)
    _check(ow, pw, x, r, act)


@pytest.mark.parametrize("m", [17, 40])
def test_prefill_rows_dense(m):
    """Dense bf16 weights: passes of 16 rows."""
    print(f"[prefill] m={m} dense bf16", flush=True)
    d, ffn = 1024, 1536
    ow, pw = generic_case((m, 16, 7), d, ffn, 16, 0)
    x = W.generic_act((m, 1), (m, d), "bf16")
    r = W.generic_act((m, 2), (m, d), "bf16")
    _check(ow, pw, x, r, "bf16")


def test_prefill_max_rows():
    """4096 rows, the most a call takes: 64 row tiles."""
    m, d, ffn = 4096, 256, 512
    print(f"[prefill] m={m} bits=4 group=64", flush=True)
    ow, pw = generic_case((m, 4, 7), d, ffn, 4, 64)
    x = W.generic_act((m, 1), (m, d), "bf16")
    r = W.generic_act((m, 2), (m, d), "bf16")
    _check(ow, pw, x, r, "bf16")


@pytest.mark.parametrize("d,ffn", [(1024, 1568), (1056, 1536)])
def test_prefill_outputs_not_a_block_multiple(d, ffn):
    """Outputs a multiple of 16 but not of 64: the last block has idle waves
    (gate/up at ffn 1568, down at d 1056; the other projection of each pair
    has a k the tiled kernel does not take and runs in passes)."""
    m = 70
    print(f"[prefill] m={m} d={d} ffn={ffn}", flush=True)
    ow, pw = generic_case((m, d, ffn), d, ffn, 8, 32)
    x = W.generic_act((m, 1), (m, d), "bf16")
    r = W.generic_act((m, 2), (m, d), "bf16")
    _check(ow, pw, x, r, "bf16")


def test_prefill_llama3_8b_shape():
    wl = W.WORKLOADS[5]
    print("[prefill] workload 5 m=128", flush=True)
    ow, pw = workload_case(5)
    x, r = W.activations(wl, 128)
    _check(ow, pw, x, r, wl.act)


def test_prefill_projection_with_bias():
    qdm = _qdm()
    m, n, k = 33, 1003, 1024
    w32 = W.generic_weights((m, n), n, k, 0.05)
    q, sb = qdm.quantize_pack_rows(w32, 8, 64)
    pw = qdm.Weight.from_host(n, k, 8, 64, q, sb)
    c, s, b = oracle.quantize_affine(w32, 8, 64)
    x = W.generic_act((m, 3), (m, k), "bf16")
    bias = W.generic_act((n, 4), (n,), "bf16", 0.1)
    y = qdm.gemv_linear(to_device(x), pw, bias=to_device(bias))
    torch.cuda.synchronize()
    ref = oracle.linear(x.values, oracle.dequantize(c, s, b, 64), bias.values)
    assert oracle.scaled_error(from_device(y), ref) <= TOL["bf16"]


def test_prefill_chain():
    qdm = _qdm()
    m, d, ffn = 20, 1024, 1536
    _, (gu, dn) = generic_case((m, 9), d, ffn, 4, 64)
    a = to_device(W.generic_act((m, 5), (m, d), "bf16"))
    b = to_device(W.generic_act((m, 6), (m, d), "bf16"))
    w = to_device(W.to_storage(np.random.default_rng(m).uniform(0.5, 1.5, d).astype(np.float32), "bf16"))
    s = torch.empty_like(a)
    y = qdm.mlp_decode_rmsnorm(a, b, w, 1e-5, gu, dn, s_out=s)
    s_u, n_u = qdm.add_rmsnorm(a, b, w, 1e-5)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    torch.cuda.synchronize()
    assert torch.equal(y, y_u) and torch.equal(s, s_u)


def test_prefill_mx_rows():
    qdm = _qdm()
    m, d, ffn = 40, 1024, 1536
    fmt = qdm.QDM_MXFP4
    g32, u32 = W.generic_weights((m, 11), ffn, d), W.generic_weights((m, 12), ffn, d)
    d32 = W.generic_weights((m, 13), d, ffn)
    q, e = qdm.quantize_mx_gate_up(g32, u32, fmt)
    gu = qdm.Weight.from_host(ffn, d, fmt, 32, q, None, block_scales=e)
    dq, de = qdm.quantize_mx(d32, fmt)
    dn = qdm.Weight.from_host(d, ffn, fmt, 32, dq, None, block_scales=de)
    deq = [oracle.dequantize_mx(*oracle.quantize_mx(a, "mxfp4"), "mxfp4") for a in (g32, u32, d32)]
    x = W.generic_act((m, 14), (m, d), "bf16")
    r = W.generic_act((m, 15), (m, d), "bf16")
    y = qdm.mlp_decode(to_device(x), to_device(r), gu, dn)
    torch.cuda.synchronize()
    _, y_ref = oracle.mlp_decode(x.values, r.values, *deq)
    assert oracle.scaled_error(from_device(y), y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("bits,group", [(8, 128), (4, 64), (4, 32), (8, 32)])
def test_prefill_sb16_rows(bits, group):
    qdm = _qdm()
    fmt = {8: qdm.QDM_U8_SB16, 4: qdm.QDM_U4_SB16}[bits]
    m, d, ffn = 90, 1024, 1536
    print(f"[prefill] m={m} sb16 bits={bits} group={group}", flush=True)
    g32, u32 = W.generic_weights((m, 21), ffn, d), W.generic_weights((m, 22), ffn, d)
    d32 = W.generic_weights((m, 23), d, ffn)
    q, sb = qdm.quantize_pack_gate_up_sb16(g32, u32, bits, group)
    gu = qdm.Weight.from_host(ffn, d, fmt, group, q, sb)
    dq, dsb = qdm.quantize_pack_rows_sb16(d32, bits, group)
    dn = qdm.Weight.from_host(d, ffn, fmt, group, dq, dsb)
    deq = []
    for a in (g32, u32, d32):
        c, s_, b = oracle.quantize_affine_bf16sb(a, bits, group)
        deq.append(oracle.dequantize_bf16sb(c, s_, b, group))
    x = W.generic_act((m, 24), (m, d), "f16")
    r = W.generic_act((m, 25), (m, d), "f16")
    xd, rd = to_device(x), to_device(r)
    h = qdm.gemv_gate_up_swiglu(xd, gu)
    y = qdm.mlp_decode(xd, rd, gu, dn)
    torch.cuda.synchronize()
    h_ref, y_ref = oracle.mlp_decode(x.values, r.values, *deq)
    assert oracle.scaled_error(from_device(h), h_ref) <= H_TOL
    assert oracle.scaled_error(from_device(y), y_ref) <= TOL["f16"]


def test_prefill_mxfp8_rows():
    qdm = _qdm()
    m, d, ffn = 100, 1024, 1536
    print(f"[prefill] m={m} mxfp8", flush=True)
    fmt = qdm.QDM_MXFP8
    g32, u32 = W.generic_weights((m, 31), ffn, d), W.generic_weights((m, 32), ffn, d)
    d32 = W.generic_weights((m, 33), d, ffn)
    q, e = qdm.quantize_mx_gate_up(g32, u32, fmt)
    gu = qdm.Weight.from_host(ffn, d, fmt, 32, q, None, block_scales=e)
    dq, de = qdm.quantize_mx(d32, fmt)
    dn = qdm.Weight.from_host(d, ffn, fmt, 32, dq, None, block_scales=de)
    deq = [oracle.dequantize_mx(*oracle.quantize_mx(a, "mxfp8"), "mxfp8") for a in (g32, u32, d32)]
    x = W.generic_act((m, 34), (m, d), "bf16")
    r = W.generic_act((m, 35), (m, d), "bf16")
    xd = to_device(x)
    h = qdm.gemv_gate_up_swiglu(xd, gu)
    y = qdm.mlp_decode(xd, to_device(r), gu, dn)
    torch.cuda.synchronize()
    h_ref, y_ref = oracle.mlp_decode(x.values, r.values, *deq)
    assert oracle.scaled_error(from_device(h), h_ref) <= H_TOL
    assert oracle.scaled_error(from_device(y), y_ref) <= TOL["bf16"]


@pytest.mark.parametrize("bits,group", [(8, 32), (4, 64)])
def test_prefill_fp32_rows_run_in_passes(bits, group):
    """fp32 activations: the tiled kernels take 16-bit rows only, so 20 fp32
    rows run as two passes of the few-row kernels; fp32 bars (1e-5) apply."""
    m, d, ffn = 20, 512, 1024
    print(f"[prefill] m={m} f32 bits={bits} group={group}", flush=True)
    ow, pw = generic_case((m, bits, group, 11), d, ffn, bits, group)
    x = W.generic_act((m, 1), (m, d), "f32")
    r = W.generic_act((m, 2), (m, d), "f32")
    _check(ow, pw, x, r, "f32")


@pytest.mark.parametrize("bits,group,d", [(4, 64, 128), (8, 64, 64), (4, 32, 128), (8, 32, 128)])
@pytest.mark.parametrize("m", [17, 65])
def test_prefill_smallest_shapes(m, bits, group, d):
    """One k-block of K (a pipeline of one iteration, no split), a single
    block of outputs (at d = 64 the down projection's block has two idle
    waves), ragged rows."""
    ffn = 128 if bits == 4 or group == 32 else 64
    print(f"[prefill] smallest m={m} bits={bits} group={group} d={d} ffn={ffn}", flush=True)
    ow, pw = generic_case((m, bits, group, d, 13), d, ffn, bits, group)
    x = W.generic_act((m, 1), (m, d), "bf16")
    r = W.generic_act((m, 2), (m, d), "bf16")
    _check(ow, pw, x, r, "bf16")
