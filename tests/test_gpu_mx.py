"""GPU parity with MXFP4 / MXFP8 block-scaled weights (one row, the
weight-streaming kernel's hardware-decoded forms) through the C ABI.

Bars: h within 1e-5 scaled error and y within 5e-3 (bf16 / f16) or 1e-5
(fp32) of the fp64 oracle on the oracle's own MX dequantization of the same
fp32 draws; the chained call bitwise equal to add + RMSNorm then the MLP;
projections on sampled rows at vocabulary size; 2..16 rows on the
matrix-core kernels; several-row projections rejected."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import H_TOL, TOL, from_device, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FMTS = {"mxfp4": 0x104, "mxfp8": 0x108}


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


def _mx_case(g32, u32, d32, name):
    qdm = _qdm()
    fmt = FMTS[name]
    ffn, d = g32.shape
    q, e = qdm.quantize_mx_gate_up(g32, u32, fmt)
    gu = qdm.Weight.from_host(ffn, d, fmt, 32, q, None, block_scales=e)
    dq, de = qdm.quantize_mx(d32, fmt)
    dn = qdm.Weight.from_host(d, ffn, fmt, 32, dq, None, block_scales=de)
    deq = [oracle.dequantize_mx(*oracle.quantize_mx(a, name), name) for a in (g32, u32, d32)]
    return deq, (gu, dn)


def _check_mlp(deq, pw, x, r, act):
    qdm = _qdm()
    gu, dn = pw
    xd, rd = to_device(x), to_device(r)
    h = qdm.gemv_gate_up_swiglu(xd, gu)
    y = qdm.mlp_decode(xd, rd, gu, dn)
    torch.cuda.synchronize()
    h_ref, y_ref = oracle.mlp_decode(x.values, r.values, *deq)
    eh = oracle.scaled_error(from_device(h), h_ref)
    ey = oracle.scaled_error(from_device(y), y_ref)
    print(f"  h err {eh:.3e}  y err {ey:.3e}", flush=True)
    assert eh <= H_TOL, eh
    assert ey <= TOL[act], ey


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("wl_index", [2, 4])
def test_mx_mlp_workload_shapes(wl_index, name):
    wl = W.WORKLOADS[wl_index]
    print(f"[mx] workload {wl_index} {name}", flush=True)
    deq, pw = _mx_case(*W.weights_f32(wl, 0), name)
    x, r = W.activations(wl, 1)
    _check_mlp(deq, pw, x, r, wl.act)


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d,ffn", [(256, 512), (1024, 2816), (2048, 1536)])
def test_mx_mlp_shapes_dtypes(d, ffn, act, name):
    print(f"[mx] d={d} ffn={ffn} act={act} {name}", flush=True)
    g32 = W.generic_weights((d, ffn, 1), ffn, d, 0.05)
    u32 = W.generic_weights((d, ffn, 2), ffn, d, 0.05)
    d32 = W.generic_weights((d, ffn, 3), d, ffn, 0.05)
    deq, pw = _mx_case(g32, u32, d32, name)
    x = W.generic_act((d, 4), (1, d), act)
    r = W.generic_act((d, 5), (1, d), act)
    _check_mlp(deq, pw, x, r, act)


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_mx_chain(name):
    qdm = _qdm()
    wl = W.WORKLOADS[4]
    print(f"[mx] chain {name}", flush=True)
    deq, (gu, dn) = _mx_case(*W.weights_f32(wl, 0), name)
    a, b, w = W.chain_inputs(wl, 1)
    ad, bd, wd = to_device(a), to_device(b), to_device(w)
    s = torch.empty_like(ad)
    y = qdm.mlp_decode_rmsnorm(ad, bd, wd, 1e-5, gu, dn, s_out=s)
    s_u, n_u = qdm.add_rmsnorm(ad, bd, wd, 1e-5)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    torch.cuda.synchronize()
    assert torch.equal(y, y_u) and torch.equal(s, s_u)
    _, _, _, y_ref = oracle.mlp_decode_rmsnorm(a.values, b.values, w.values, 1e-5, wl.act, *deq)
    e = oracle.scaled_error(from_device(y), y_ref)
    print(f"  y err {e:.3e}", flush=True)
    assert e <= TOL[wl.act]


@pytest.mark.parametrize("name", ["mxfp4", "mxfp8"])
def test_mx_vocab_projection(name):
    qdm = _qdm()
    p = W.PROJECTIONS["qwen3_8b_lm_head"]
    print(f"[mx] lm_head {name}", flush=True)
    fmt = FMTS[name]
    w32, _, x = W.projection_inputs(p, 1)
    qq, e = qdm.quantize_mx(w32, fmt)
    pw = qdm.Weight.from_host(p.n, p.k, fmt, 32, qq, None, block_scales=e)
    y = qdm.gemv_linear(to_device(x), pw)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, p.n - 1], np.random.default_rng(5).choice(p.n, 2048, replace=False)]))
    ref = oracle.linear(x.values, oracle.dequantize_mx(*oracle.quantize_mx(w32[rows], name), name))
    err = oracle.scaled_error(from_device(y)[:, rows], ref)
    print(f"  sampled err {err:.3e}", flush=True)
    assert err <= TOL[p.act]


@pytest.mark.parametrize("name", ["mxfp4", "mxfp8"])
def test_mx_projection_with_bias(name):
    qdm = _qdm()
    n, k = 1003, 1536
    fmt = FMTS[name]
    w32 = W.generic_weights((n, k, fmt), n, k, 0.05)
    qq, e = qdm.quantize_mx(w32, fmt)
    pw = qdm.Weight.from_host(n, k, fmt, 32, qq, None, block_scales=e)
    x = W.generic_act((k, 1), (1, k), "bf16")
    b = W.generic_act((n, 3), (n,), "bf16", 0.1)
    y = qdm.gemv_linear(to_device(x), pw, bias=to_device(b))
    torch.cuda.synchronize()
    ref = oracle.linear(x.values, oracle.dequantize_mx(*oracle.quantize_mx(w32, name), name), b.values)
    assert oracle.scaled_error(from_device(y), ref) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("m", [2, 4, 16])
def test_mx_rows(m, act, name):
    """Several rows on the matrix-core kernels: elements converted to exact
    operands, the block scale folded per 32-wide chunk."""
    print(f"[mx] rows m={m} act={act} {name}", flush=True)
    d, ffn = 1024, 1536
    g32 = W.generic_weights((m, 1), ffn, d, 0.05)
    u32 = W.generic_weights((m, 2), ffn, d, 0.05)
    d32 = W.generic_weights((m, 3), d, ffn, 0.05)
    deq, pw = _mx_case(g32, u32, d32, name)
    x = W.generic_act((m, 4), (m, d), act)
    r = W.generic_act((m, 5), (m, d), act)
    _check_mlp(deq, pw, x, r, act)


@pytest.mark.parametrize("m", [4, 16])
@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_mx_rows_llama3_8b_shape(name, m):
    wl = W.WORKLOADS[5]
    print(f"[mx] workload 5 m={m} {name}", flush=True)
    deq, pw = _mx_case(*W.weights_f32(wl, 0), name)
    x, r = W.activations(wl, m)
    _check_mlp(deq, pw, x, r, wl.act)


def test_mx_rows_chain():
    """The chain at 4 rows with MX weights: bitwise equal to the three launches."""
    qdm = _qdm()
    print("[mx] rows chain m=4 mxfp4", flush=True)
    m, d, ffn = 4, 1024, 1536
    _, (gu, dn) = _mx_case(W.generic_weights((9, 1), ffn, d), W.generic_weights((9, 2), ffn, d),
                           W.generic_weights((9, 3), d, ffn), "mxfp4")
    a = to_device(W.generic_act((9, 4), (m, d), "bf16"))
    b = to_device(W.generic_act((9, 5), (m, d), "bf16"))
    w = to_device(W.to_storage(np.random.default_rng(9).uniform(0.5, 1.5, d).astype(np.float32), "bf16"))
    s = torch.empty_like(a)
    y = qdm.mlp_decode_rmsnorm(a, b, w, 1e-5, gu, dn, s_out=s)
    s_u, n_u = qdm.add_rmsnorm(a, b, w, 1e-5)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    torch.cuda.synchronize()
    assert torch.equal(y, y_u) and torch.equal(s, s_u)


def test_mx_rows_projection_rejected():
    """Projections with MX weights take one row only."""
    qdm = _qdm()
    n, k = 256, 512
    qq, e = qdm.quantize_mx(W.generic_weights((1,), n, k), qdm.QDM_MXFP8)
    pw = qdm.Weight.from_host(n, k, qdm.QDM_MXFP8, 32, qq, None, block_scales=e)
    x = to_device(W.generic_act((1,), (4, k), "bf16"))
    with pytest.raises(qdm.QdmError) as ei:
        qdm.gemv_linear(x, pw)
    assert ei.value.status == qdm.QDM_ERR_UNSUPPORTED
