"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: max|out - ref| / max|ref| <= 1e-5 for fp32 outputs (and for the fp32
hidden row h), <= 5e-3 for bf16 / f16 outputs; s of add+RMSNorm bitwise
equal to a + b rounded once; x = 0 and all-zero down weights give y == r
bitwise; repeated calls are bitwise identical.
Workloads are the five synthetic LLM-shaped MLPs at full size plus small
ragged shapes; rows m in {1, 2, 3, 4, 5, 16}."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import (H_TOL, TOL, from_device, generic_case, product_weights_from_f32,
                       to_device, workload_case)

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


def _acts(wl_index, m, set_index=0, dtype=None):
    wl = W.WORKLOADS[wl_index]
    x, r = W.activations(wl, m, set_index)
    if dtype is not None and dtype != wl.act:
        x, r = W.to_storage(x.values, dtype), W.to_storage(r.values, dtype)
    return x, r


def _check_mlp(ow, pw, x, r, tol):
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
    assert ey <= tol, ey
    return y


# ------------------------------------------------------------------ the five workloads, full size

@pytest.mark.parametrize("wl_index", [1, 2, 3])
def test_workload_mlp(wl_index):
    ow, pw = workload_case(wl_index)
    x, r = _acts(wl_index, 1)
    _check_mlp(ow, pw, x, r, TOL[W.WORKLOADS[wl_index].act])


@pytest.mark.parametrize("set_index", [0, 17, 35])
def test_workload4_sets(set_index):
    ow, pw = workload_case(4, set_index)
    x, r = _acts(4, 1, set_index)
    _check_mlp(ow, pw, x, r, TOL["bf16"])


@pytest.mark.parametrize("m", [1, 4, 16])
def test_workload5_rows(m):
    ow, pw = workload_case(5)
    x, r = _acts(5, m)
    _check_mlp(ow, pw, x, r, TOL["bf16"])


def test_holdout_seed_workload2():
    """A weight set and activations never used while tuning."""
    ow, pw = workload_case(2, 7)
    x, r = _acts(2, 1, set_index=7)
    _check_mlp(ow, pw, x, r, TOL["bf16"])


# ------------------------------------------------------------------ kernels one at a time

@pytest.mark.parametrize("wl_index", [1, 2, 5])
def test_down_residual_alone(wl_index):
    """The down kernel fed the oracle's own hidden row (rounded to fp32)."""
    qdm = _qdm()
    ow, (gu, dn) = workload_case(wl_index)
    x, r = _acts(wl_index, 1)
    _, _, h_ref = oracle.gate_up_swiglu(x.values, ow.wg, ow.wu)
    h32 = h_ref.astype(np.float32)
    y = qdm.gemv_down_residual(torch.from_numpy(h32).cuda(), to_device(r), dn)
    y_ref = oracle.down_residual(h32, r.values, ow.wd)
    e = oracle.scaled_error(from_device(y), y_ref)
    print(f"  y err {e:.3e}", flush=True)
    assert e <= TOL[W.WORKLOADS[wl_index].act]


# ------------------------------------------------------------------ shapes, rows, dtypes

SHAPES = [
    # d, ffn, bits, group: ragged K tiles (row bytes not a multiple of 1 KiB), small and odd sizes
    (96, 160, 8, 32),
    (160, 96, 4, 32),
    (224, 352, 8, 32),
    (1152, 640, 4, 64),
    (384, 1408, 8, 128),
    (2176, 384, 4, 128),
    (104, 200, 16, 0),
    (1544, 264, 16, 0),
]


@pytest.mark.parametrize("d,ffn,bits,group", SHAPES)
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
def test_shapes_and_dtypes(d, ffn, bits, group, act):
    ow, pw = generic_case((d, ffn, bits), d, ffn, bits, group)
    x = W.generic_act((d, 4), (1, d), act)
    r = W.generic_act((d, 5), (1, d), act)
    _check_mlp(ow, pw, x, r, TOL[act])


@pytest.mark.parametrize("m", [2, 3, 4, 5, 16])
@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32), (16, 0), (4, 128)])
def test_rows(m, bits, group):
    """2..16 rows: bf16 activations take the matrix-core kernels."""
    d, ffn = 384, 640
    ow, pw = generic_case((m, bits), d, ffn, bits, group)
    x = W.generic_act((m, 4), (m, d), "bf16")
    r = W.generic_act((m, 5), (m, d), "bf16")
    _check_mlp(ow, pw, x, r, TOL["bf16"])


@pytest.mark.parametrize("m", [2, 7, 16])
@pytest.mark.parametrize("bits,group", [(8, 64), (8, 32), (4, 32), (16, 0), (4, 128)])
def test_rows_persistent_gate_up(m, bits, group):
    """K = 1024 splits evenly over the persistent matrix-core gate/up kernel's
    waves for every format (its k-block is 32..128 codes); ffn = 896 is 56
    tiles of 16 (a multiple of every group size)."""
    d, ffn = 1024, 896
    ow, pw = generic_case((m, bits, 1), d, ffn, bits, group)
    x = W.generic_act((m, 6), (m, d), "bf16")
    r = W.generic_act((m, 7), (m, d), "bf16")
    _check_mlp(ow, pw, x, r, TOL["bf16"])


@pytest.mark.parametrize("m", [3, 16])
@pytest.mark.parametrize("act", ["f16", "f32"])
@pytest.mark.parametrize("bits,group", [(8, 32), (4, 64)])
def test_rows_other_dtypes(m, act, bits, group):
    """f16 activations: vector gate/up, matrix-core down; fp32: vector both."""
    d, ffn = 256, 512
    ow, pw = generic_case((m, bits, len(act)), d, ffn, bits, group)
    x = W.generic_act((m, 6), (m, d), act)
    r = W.generic_act((m, 7), (m, d), act)
    _check_mlp(ow, pw, x, r, TOL[act])


def test_rows_ragged_tiles_fall_back():
    """Output widths that are not whole 16-wide tiles use the vector kernel."""
    d, ffn = 104, 200
    ow, pw = generic_case((55,), d, ffn, 16, 0)
    x = W.generic_act((55, 1), (5, d), "bf16")
    r = W.generic_act((55, 2), (5, d), "bf16")
    _check_mlp(ow, pw, x, r, TOL["bf16"])


@pytest.mark.parametrize("bits,group", [(8, 32), (16, 0)])
def test_rows_are_independent(bits, group):
    """Within one m-row call rows do not interact: permuting the input rows
    permutes the output rows bitwise, and changing one input row changes only
    that output row."""
    qdm = _qdm()
    d, ffn, m = 256, 512, 6
    _, (gu, dn) = generic_case((77, bits), d, ffn, bits, group)
    x = to_device(W.generic_act((7, 1), (m, d), "bf16"))
    r = to_device(W.generic_act((7, 2), (m, d), "bf16"))
    y = qdm.mlp_decode(x, r, gu, dn)
    p = torch.tensor([3, 0, 5, 1, 4, 2], device="cuda")
    yp = qdm.mlp_decode(x[p].contiguous(), r[p].contiguous(), gu, dn)
    assert torch.equal(yp, y[p])
    x2 = x.clone()
    x2[4] = -x2[4]
    y2 = qdm.mlp_decode(x2, r, gu, dn)
    keep = [0, 1, 2, 3, 5]
    assert torch.equal(y2[keep], y[keep])
    assert not torch.equal(y2[4], y[4])


# ------------------------------------------------------------------ special cases (bitwise)

@pytest.mark.parametrize("m", [4, 16])
@pytest.mark.parametrize("bits,group", [(4, 64), (8, 128)])
def test_rows_graph_replay(m, bits, group):
    """A few-row MLP captured into a HIP graph after one eager call replays
    bitwise equal to the eager result, with other work between replays, and
    meets the oracle bar."""
    qdm = _qdm()
    d, ffn = 1024, 1536
    ow, (gu, dn) = generic_case((91, bits, m), d, ffn, bits, group)
    x = W.generic_act((m, 8), (m, d), "bf16")
    r = W.generic_act((m, 9), (m, d), "bf16")
    xd, rd = to_device(x), to_device(r)
    ws = torch.empty(qdm.mlp_workspace_bytes(m, qdm.QDM_BF16, gu, dn), dtype=torch.uint8, device="cuda")
    y_eager = qdm.mlp_decode(xd, rd, gu, dn, workspace=ws).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(rd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qdm.mlp_decode(xd, rd, gu, dn, workspace=ws, out=out)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y_eager)
    _, y_ref = oracle.mlp_decode(x.values, r.values, ow.wg, ow.wu, ow.wd)
    ey = oracle.scaled_error(from_device(out), y_ref)
    print(f"  y err {ey:.3e}", flush=True)
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("wl_index", [1, 2, 5])
def test_zero_input_gives_residual(wl_index):
    qdm = _qdm()
    _, (gu, dn) = workload_case(wl_index)
    _, r = _acts(wl_index, 1)
    rd = to_device(r)
    y = qdm.mlp_decode(torch.zeros_like(rd), rd, gu, dn)
    assert torch.equal(y, rd)


def test_zero_down_weights_give_residual():
    qdm = _qdm()
    d, ffn = 256, 512
    g32 = W.generic_weights((3, 1), ffn, d)
    u32 = W.generic_weights((3, 2), ffn, d)
    gu, dn = product_weights_from_f32(g32, u32, np.zeros((d, ffn), np.float32), 8, 32)
    x = to_device(W.generic_act((3, 4), (1, d), "f32"))
    r = to_device(W.generic_act((3, 5), (1, d), "f32"))
    assert torch.equal(qdm.mlp_decode(x, r, gu, dn), r)


def test_deterministic():
    qdm = _qdm()
    _, (gu, dn) = workload_case(2)
    x, r = _acts(2, 1)
    xd, rd = to_device(x), to_device(r)
    y1 = qdm.mlp_decode(xd, rd, gu, dn).clone()
    for _ in range(3):
        assert torch.equal(qdm.mlp_decode(xd, rd, gu, dn), y1)


# ------------------------------------------------------------------ metamorphic

def test_ffn_permutation_invariance():
    """Permuting the hidden units (gate/up rows and the matching W_down columns)
    leaves y unchanged up to summation order.  W_down columns move by whole
    groups, so every group keeps its quantization."""
    qdm = _qdm()
    d, ffn, g = 512, 768, 64
    g32 = W.generic_weights((9, 1), ffn, d)
    u32 = W.generic_weights((9, 2), ffn, d)
    d32 = W.generic_weights((9, 3), d, ffn)
    perm = (np.random.default_rng(10).permutation(ffn // g)[:, None] * g + np.arange(g)).reshape(-1)
    a = product_weights_from_f32(g32, u32, d32, 8, g)
    b = product_weights_from_f32(np.ascontiguousarray(g32[perm]), np.ascontiguousarray(u32[perm]),
                                 np.ascontiguousarray(d32[:, perm]), 8, g)
    x = to_device(W.generic_act((9, 4), (1, d), "f32"))
    r = to_device(W.generic_act((9, 5), (1, d), "f32"))
    ya = from_device(qdm.mlp_decode(x, r, *a))
    yb = from_device(qdm.mlp_decode(x, r, *b))
    assert oracle.scaled_error(yb, ya) <= 1e-5


def test_residual_shift():
    qdm = _qdm()
    _, (gu, dn) = workload_case(1)
    x, r = _acts(1, 1)
    xd, rd = to_device(x), to_device(r)
    delta = torch.linspace(-1, 1, rd.numel(), device="cuda").reshape(rd.shape)
    y0 = from_device(qdm.mlp_decode(xd, rd, gu, dn))
    y1 = from_device(qdm.mlp_decode(xd, rd + delta, gu, dn))
    assert np.allclose(y1 - y0, from_device(delta), atol=1e-5)


# ------------------------------------------------------------------ add + RMSNorm

def _check_rmsnorm(a, b, w, eps, dtype):
    qdm = _qdm()
    s, n = qdm.add_rmsnorm(to_device(a), to_device(b), to_device(w), eps)
    torch.cuda.synchronize()
    s_ref, n_ref = oracle.add_rmsnorm(a.values, b.values, w.values, eps, dtype)
    assert np.array_equal(from_device(s), s_ref)
    e = oracle.scaled_error(from_device(n), n_ref)
    print(f"  n err {e:.3e}", flush=True)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("wl_index", [1, 2])
def test_workload_add_rmsnorm(wl_index):
    wl = W.WORKLOADS[wl_index]
    a, b, w = W.rmsnorm_inputs(wl)
    _check_rmsnorm(a, b, w, wl.norm_eps, wl.norm_dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rows,n", [(1, 1), (1, 255), (3, 4096), (2, 5000), (1, 14336)])
def test_add_rmsnorm_shapes(dtype, rows, n):
    a = W.generic_act((n, 1), (rows, n), dtype)
    b = W.generic_act((n, 2), (rows, n), dtype)
    w = W.to_storage(np.random.default_rng(n).uniform(0.5, 1.5, n).astype(np.float32), dtype)
    _check_rmsnorm(a, b, w, 1e-5, dtype)


def test_add_rmsnorm_zero_row():
    a = W.to_storage(np.zeros((1, 512), np.float32), "f16")
    w = W.to_storage(np.ones(512, np.float32), "f16")
    _check_rmsnorm(a, a, w, 1e-5, "f16")


def test_add_rmsnorm_in_place_sum():
    """s_out may alias a."""
    qdm = _qdm()
    a = W.generic_act((5, 1), (1, 2048), "f16")
    b = W.generic_act((5, 2), (1, 2048), "f16")
    w = W.to_storage(np.ones(2048, np.float32), "f16")
    ad = to_device(a)
    s, n = qdm.add_rmsnorm(ad, to_device(b), to_device(w), 1e-5, s_out=ad)
    s_ref, _ = oracle.add_rmsnorm(a.values, b.values, w.values, 1e-5, "f16")
    assert np.array_equal(from_device(ad), s_ref)

