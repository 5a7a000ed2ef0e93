"""GPU parity with the affine formats whose (scale, bias) pairs are bf16
(QDM_U8_SB16 / QDM_U4_SB16) through the C ABI: one row on the streaming
kernel, 2..16 rows on the matrix-core kernels, the chain and a projection.

Bars: h within 1e-5 and y within 5e-3 (bf16) scaled error of the fp64
oracle on its own bf16-pair quantization of the same fp32 draws; the chain
bitwise equal to add + RMSNorm then the MLP."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_cases import H_TOL, TOL, from_device, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FMT = {8: 0x208, 4: 0x204}


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


def _case(g32, u32, d32, bits, group):
    qdm = _qdm()
    ffn, d = g32.shape
    q, sb = qdm.quantize_pack_gate_up_sb16(g32, u32, bits, group)
    gu = qdm.Weight.from_host(ffn, d, FMT[bits], group, q, sb)
    dq, dsb = qdm.quantize_pack_rows_sb16(d32, bits, group)
    dn = qdm.Weight.from_host(d, ffn, FMT[bits], group, dq, dsb)
    deq = []
    for a in (g32, u32, d32):
        c, s, b = oracle.quantize_affine_bf16sb(a, bits, group)
        deq.append(oracle.dequantize_bf16sb(c, s, b, group))
    return deq, (gu, dn)


def _check(deq, pw, x, r, act):
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


@pytest.mark.parametrize("wl_index", [2, 4, 5])
def test_sb16_workload_shapes(wl_index):
    wl = W.WORKLOADS[wl_index]
    print(f"[sb16] workload {wl_index} m=1", flush=True)
    deq, pw = _case(*W.weights_f32(wl, 0), wl.bits, wl.group)
    x, r = W.activations(wl, 1)
    _check(deq, pw, x, r, wl.act)


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32), (4, 128), (8, 128), (8, 32)])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_sb16_rows(m, bits, group, act):
    print(f"[sb16] m={m} bits={bits} group={group} act={act}", flush=True)
    d, ffn = 1024, 1536
    deq, pw = _case(W.generic_weights((m, bits, 1), ffn, d, 0.05), W.generic_weights((m, bits, 2), ffn, d, 0.05),
                    W.generic_weights((m, bits, 3), d, ffn, 0.05), bits, group)
    x = W.generic_act((m, 4), (m, d), act)
    r = W.generic_act((m, 5), (m, d), act)
    _check(deq, pw, x, r, act)


@pytest.mark.parametrize("m", [1, 4])
def test_sb16_chain(m):
    qdm = _qdm()
    d, ffn = 1024, 1536
    _, (gu, dn) = _case(W.generic_weights((m, 7), ffn, d), W.generic_weights((m, 8), ffn, d),
                        W.generic_weights((m, 9), d, ffn), 4, 64)
    a = to_device(W.generic_act((m, 10), (m, d), "bf16"))
    b = to_device(W.generic_act((m, 11), (m, d), "bf16"))
    w = to_device(W.to_storage(np.random.default_rng(m).uniform(0.5, 1.5, d).astype(np.float32), "bf16"))
    s = torch.empty_like(a)
    y = qdm.mlp_decode_rmsnorm(a, b, w, 1e-5, gu, dn, s_out=s)
    s_u, n_u = qdm.add_rmsnorm(a, b, w, 1e-5)
    y_u = qdm.mlp_decode(n_u, s_u, gu, dn)
    torch.cuda.synchronize()
    assert torch.equal(y, y_u) and torch.equal(s, s_u)


def test_sb16_projection():
    qdm = _qdm()
    n, k = 1003, 2048
    w32 = W.generic_weights((n, k), n, k, 0.05)
    q, sb = qdm.quantize_pack_rows_sb16(w32, 8, 128)
    pw = qdm.Weight.from_host(n, k, FMT[8], 128, q, sb)
    c, s, b = oracle.quantize_affine_bf16sb(w32, 8, 128)
    x = W.generic_act((k, 1), (1, k), "bf16")
    bias = W.generic_act((n, 2), (n,), "bf16", 0.1)
    y = qdm.gemv_linear(to_device(x), pw, bias=to_device(bias))
    torch.cuda.synchronize()
    ref = oracle.linear(x.values, oracle.dequantize_bf16sb(c, s, b, 128), bias.values)
    assert oracle.scaled_error(from_device(y), ref) <= TOL["bf16"]


def test_sb16_fp32_rows_rejected():
    """Several fp32 rows: the matrix-core kernels take 16-bit activations only."""
    qdm = _qdm()
    d, ffn = 256, 512
    _, (gu, dn) = _case(W.generic_weights((1,), ffn, d), W.generic_weights((2,), ffn, d),
                        W.generic_weights((3,), d, ffn), 8, 64)
    x = to_device(W.generic_act((1,), (3, d), "f32"))
    with pytest.raises(qdm.QdmError) as ei:
        qdm.mlp_decode(x, x.clone(), gu, dn)
    assert ei.value.status == qdm.QDM_ERR_UNSUPPORTED
