"""GPU parity of the decode chain (add + RMSNorm feeding the MLP, the sum as
its residual) through the C ABI.

Bars: s bitwise equal to the oracle's a + b rounded once; the output within
the MLP's tolerance of the oracle chain (5e-3 scaled for bf16 / f16, 1e-5
for fp32); and the chained call bitwise equal to add + RMSNorm followed by
the MLP from the same library (the one-row form recomputes the norm in every
gate/up block with the standalone kernel's rounding and summation order).
Inputs: a, b ~ N(0,1), norm weight ~ U(0.5, 1.5), in each workload's
activation dtype, at the five workloads' full sizes."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import TOL, from_device, generic_case, to_device, workload_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EPS = 1e-5


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


def _chain_check(ow, pw, a, b, w, dtype):
    qdm = _qdm()
    gu, dn = pw
    ad, bd, wd = to_device(a), to_device(b), to_device(w)
    s_f = torch.empty_like(ad)
    y_f = qdm.mlp_decode_rmsnorm(ad, bd, wd, EPS, gu, dn, s_out=s_f)
    s_u, n_u = qdm.add_rmsnorm(ad, bd, wd, EPS)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    torch.cuda.synchronize()
    assert torch.equal(s_f, s_u)
    assert torch.equal(y_f, y_u), "chained call differs from add + RMSNorm then MLP"
    s_ref, _, _, y_ref = oracle.mlp_decode_rmsnorm(a.values, b.values, w.values, EPS, dtype, ow.wg, ow.wu, ow.wd)
    assert np.array_equal(from_device(s_f), s_ref)
    e = oracle.scaled_error(from_device(y_f), y_ref)
    print(f"  y err {e:.3e}", flush=True)
    assert e <= TOL[dtype], e
    return y_f


@pytest.mark.parametrize("wl_index", [1, 2, 3, 4])
def test_workload_chain(wl_index):
    wl = W.WORKLOADS[wl_index]
    print(f"[chain] workload {wl_index} m=1", flush=True)
    ow, pw = workload_case(wl_index)
    a, b, w = W.chain_inputs(wl, 1)
    _chain_check(ow, pw, a, b, w, wl.act)


@pytest.mark.parametrize("m", [1, 4, 16])
def test_workload5_chain_rows(m):
    """Llama-3-8B 4-bit: one row on the chained streaming kernels, several rows
    on the chained matrix-core kernels."""
    wl = W.WORKLOADS[5]
    print(f"[chain] workload 5 m={m}", flush=True)
    ow, pw = workload_case(5)
    a, b, w = W.chain_inputs(wl, m)
    _chain_check(ow, pw, a, b, w, wl.act)


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d,ffn,bits,group", [(512, 1536, 8, 32), (1024, 2048, 4, 128), (768, 1280, 16, 0),
                                              (2048, 5632, 8, 64)])
def test_chain_shapes_and_dtypes(d, ffn, bits, group, act):
    print(f"[chain] d={d} ffn={ffn} bits={bits} group={group} act={act}", flush=True)
    ow, pw = generic_case(d + ffn, d, ffn, bits, group)
    a = W.generic_act((d, 11), (1, d), act)
    b = W.generic_act((d, 12), (1, d), act)
    w = W.to_storage(np.random.default_rng(d).uniform(0.5, 1.5, d).astype(np.float32), act)
    _chain_check(ow, pw, a, b, w, act)


def test_chain_in_place():
    """s_out may alias a and out may alias b; with s_out omitted s is not written."""
    qdm = _qdm()
    wl = W.WORKLOADS[2]
    ow, (gu, dn) = workload_case(2)
    a, b, w = W.chain_inputs(wl, 1)
    ad, bd, wd = to_device(a), to_device(b), to_device(w)
    s_u, n_u = qdm.add_rmsnorm(ad, bd, wd, EPS)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    y_plain = qdm.mlp_decode_rmsnorm(ad, bd, wd, EPS, gu, dn)
    a2, b2 = ad.clone(), bd.clone()
    qdm.mlp_decode_rmsnorm(a2, b2, wd, EPS, gu, dn, s_out=a2, out=b2)
    torch.cuda.synchronize()
    assert torch.equal(y_plain, y_u)
    assert torch.equal(a2, s_u) and torch.equal(b2, y_u)


def test_chain_zero_norm_weight_gives_sum():
    """A zero norm weight makes the MLP input zero: out == s bitwise."""
    qdm = _qdm()
    wl = W.WORKLOADS[4]
    _, (gu, dn) = workload_case(4)
    a, b, _ = W.chain_inputs(wl, 1)
    ad, bd = to_device(a), to_device(b)
    wz = torch.zeros(wl.d, dtype=ad.dtype, device="cuda")
    s = torch.empty_like(ad)
    y = qdm.mlp_decode_rmsnorm(ad, bd, wz, EPS, gu, dn, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(y, s)
    assert np.array_equal(from_device(s), oracle.round_to_dtype(a.values.astype(np.float64) + b.values, wl.act))


def test_chain_graph_replay():
    """The one-row chain captured in a HIP graph: every replay bitwise equal to
    the eager call (outputs cleared between replays)."""
    qdm = _qdm()
    wl = W.WORKLOADS[4]
    _, (gu, dn) = workload_case(4)
    a, b, w = W.chain_inputs(wl, 1)
    ad, bd, wd = to_device(a), to_device(b), to_device(w)
    ws = torch.empty(qdm.mlp_rmsnorm_workspace_bytes(1, qdm.QDM_BF16, gu, dn), dtype=torch.uint8, device="cuda")
    out, s = torch.empty_like(ad), torch.empty_like(ad)
    eager = qdm.mlp_decode_rmsnorm(ad, bd, wd, EPS, gu, dn, workspace=ws, s_out=s).clone()
    s_eager = s.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qdm.mlp_decode_rmsnorm(ad, bd, wd, EPS, gu, dn, workspace=ws, s_out=s, out=out)
    for _ in range(3):
        out.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager) and torch.equal(s, s_eager)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32), (4, 128)])
@pytest.mark.parametrize("m", [2, 7, 16])
def test_chain_rows(m, bits, group, act):
    """Several rows: the norm rebuilt in every matrix-core gate/up block, s
    through the workspace; bitwise equal to the three launches."""
    print(f"[chain] rows m={m} bits={bits} group={group} act={act}", flush=True)
    d, ffn = 1024, 1536
    ow, pw = generic_case((d, m, bits), d, ffn, bits, group)
    a = W.generic_act((m, 21), (m, d), act)
    b = W.generic_act((m, 22), (m, d), act)
    w = W.to_storage(np.random.default_rng(m).uniform(0.5, 1.5, d).astype(np.float32), act)
    _chain_check(ow, pw, a, b, w, act)


def test_chain_rows_in_place_and_graph():
    """Several rows with s_out aliasing a and out aliasing b, then the same
    call captured in a graph and replayed: bitwise equal to the three launches."""
    qdm = _qdm()
    m, d, ffn = 4, 1024, 1536
    _, (gu, dn) = generic_case((d, m, 99), d, ffn, 4, 64)
    a = to_device(W.generic_act((m, 31), (m, d), "bf16"))
    b = to_device(W.generic_act((m, 32), (m, d), "bf16"))
    w = to_device(W.to_storage(np.random.default_rng(3).uniform(0.5, 1.5, d).astype(np.float32), "bf16"))
    s_u, n_u = qdm.add_rmsnorm(a, b, w, EPS)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    a2, b2 = a.clone(), b.clone()
    qdm.mlp_decode_rmsnorm(a2, b2, w, EPS, gu, dn, s_out=a2, out=b2)
    torch.cuda.synchronize()
    assert torch.equal(a2, s_u) and torch.equal(b2, y_u)
    ws = torch.empty(qdm.mlp_rmsnorm_workspace_bytes(m, qdm.QDM_BF16, gu, dn), dtype=torch.uint8, device="cuda")
    out, s = torch.empty_like(a), torch.empty_like(a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qdm.mlp_decode_rmsnorm(a, b, w, EPS, gu, dn, workspace=ws, s_out=s, out=out)
    for _ in range(3):
        out.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_u) and torch.equal(s, s_u)
