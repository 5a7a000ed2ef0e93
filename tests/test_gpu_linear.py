"""GPU parity of the one-row decode projections (qdm_gemv_linear): the
vocabulary map and the attention q/k/v/o with biases, through the C ABI.

Bars: 5e-3 scaled error for bf16 / f16 outputs and 1e-5 for fp32 against the
fp64 oracle; x = 0 gives the bias bitwise; a one-row fp32 projection with a
bias is bitwise the down projection's residual form on the same kernel.
Vocabulary maps run at full size (Qwen3-8B lm_head 151936 x 4096, Llama-3.2-1B
tied embedding 128256 x 2048) and are checked on a seeded sample of output
rows that the oracle computes from those rows' own weights (quantization
groups lie within a row)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import TOL, from_device, to_device

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


def _product_weight(w32, bits, group):
    qdm = _qdm()
    n, k = w32.shape
    if bits == 16:
        return qdm.Weight.from_host(n, k, 16, 0, W.to_storage(w32, "bf16").raw, None)
    q, sb = qdm.quantize_pack_rows(w32, bits, group)
    return qdm.Weight.from_host(n, k, bits, group, q, sb)


def _oracle_weight(w32, bits, group):
    if bits == 16:
        return oracle.dequantize_dense_bf16(W.to_storage(w32, "bf16").raw)
    c, s, b = oracle.quantize_affine(w32, bits, group)
    return oracle.dequantize(c, s, b, group)


@pytest.mark.parametrize("key", ["qwen3_8b_lm_head", "llama32_1b_tied_embedding"])
def test_vocab_projection_full_size(key):
    qdm = _qdm()
    p = W.PROJECTIONS[key]
    print(f"[linear] {key} n={p.n} k={p.k}", flush=True)
    w32, _, x = W.projection_inputs(p, 1)
    pw = _product_weight(w32, p.bits, p.group)
    y = qdm.gemv_linear(to_device(x), pw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(p.seed_id)
    rows = np.unique(np.concatenate([[0, p.n - 1], rng.choice(p.n, 2048, replace=False)]))
    ref = oracle.linear(x.values, _oracle_weight(w32[rows], p.bits, p.group))
    got = from_device(y)[:, rows]
    e = oracle.scaled_error(got, ref)
    print(f"  sampled {rows.size} rows: err {e:.3e}", flush=True)
    assert e <= TOL[p.act], e


@pytest.mark.parametrize("m", [1, 4])
def test_attention_projections(m):
    qdm = _qdm()
    for key in ("qwen25_1p5b_q", "qwen25_1p5b_k", "qwen25_1p5b_v", "qwen25_1p5b_o"):
        p = W.PROJECTIONS[key]
        print(f"[linear] {key} m={m}", flush=True)
        w32, b, x = W.projection_inputs(p, m)
        pw = _product_weight(w32, p.bits, p.group)
        y = qdm.gemv_linear(to_device(x), pw, bias=None if b is None else to_device(b))
        torch.cuda.synchronize()
        ref = oracle.linear(x.values, _oracle_weight(w32, p.bits, p.group), None if b is None else b.values)
        e = oracle.scaled_error(from_device(y), ref)
        print(f"  err {e:.3e}", flush=True)
        assert e <= TOL[p.act], e


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits,group", [(8, 32), (4, 64), (8, 128), (16, 0)])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_linear_shapes(m, bits, group, act):
    """A ragged output count (1003) and both bias forms."""
    qdm = _qdm()
    n, k = 1003, 1024
    print(f"[linear] n={n} k={k} bits={bits} group={group} act={act} m={m}", flush=True)
    w32 = W.generic_weights((n, k, bits), n, k, 0.05)
    x = W.generic_act((k, m, 1), (m, k), act)
    b = W.generic_act((n, 2), (n,), act, 0.1)
    pw = _product_weight(w32, bits, group)
    wref = _oracle_weight(w32, bits, group)
    xd = to_device(x)
    for bias in (None, b):
        y = qdm.gemv_linear(xd, pw, bias=None if bias is None else to_device(bias))
        torch.cuda.synchronize()
        ref = oracle.linear(x.values, wref, None if bias is None else bias.values)
        e = oracle.scaled_error(from_device(y), ref)
        print(f"  bias={bias is not None} err {e:.3e}", flush=True)
        assert e <= TOL[act], e


@pytest.mark.parametrize("m", [1, 5])
def test_zero_input_gives_bias(m):
    qdm = _qdm()
    p = W.PROJECTIONS["qwen25_1p5b_q"]
    w32, b, _ = W.projection_inputs(p, 1)
    pw = _product_weight(w32, p.bits, p.group)
    bd = to_device(b)
    y = qdm.gemv_linear(torch.zeros((m, p.k), dtype=bd.dtype, device="cuda"), pw, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(y, bd.expand(m, -1))


def test_one_row_linear_is_the_down_form():
    """fp32, one row: the projection with bias r is bitwise the down
    projection's out = r + h W^T on the same streaming kernel."""
    qdm = _qdm()
    n, k = 2048, 4096
    w32 = W.generic_weights((7, 7), n, k, 0.02)
    pw = _product_weight(w32, 8, 64)
    h = to_device(W.generic_act((7, 8), (1, k), "f32"))
    r = to_device(W.generic_act((7, 9), (1, n), "f32"))
    y_lin = qdm.gemv_linear(h, pw, bias=r.view(-1))
    y_dn = qdm.gemv_down_residual(h, r, pw)
    torch.cuda.synchronize()
    assert torch.equal(y_lin, y_dn)
