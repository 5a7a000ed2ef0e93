"""The allocation-free MLP entry point (qdm_mlp_decode_noalloc) through the C
ABI against the ordinary one (qdm_mlp_decode, caller's workspace): bitwise
equal outputs on two calls in a row, the second with fewer rows (the fixed
array keeps the first call's contents), both within the oracle bar; a call
too large for the array is refused before anything runs."""
import ctypes

import pytest

import oracle
import workloads as W
from gpu_cases import TOL, from_device, generic_case, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU")
    import quantized_decode_mlp_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


def _call_noalloc(qdm, xd, rd, gu, dn, out):
    m = xd.shape[0]
    st = qdm._lib.qdm_mlp_decode_noalloc(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(rd.data_ptr()), m,
                                         qdm.QDM_BF16, ctypes.byref(gu.descriptor), ctypes.byref(dn.descriptor),
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("bits,group,rows", [(4, 64, (16, 4)), (8, 128, (16, 1)), (4, 64, (5, 1))])
def test_noalloc_matches_workspace_entry(bits, group, rows):
    import quantized_decode_mlp_amd as qdm
    d, ffn = 4096, 14336 if bits == 4 else 12288
    ow, (gu, dn) = generic_case((61, bits, group), d, ffn, bits, group, sigma=0.02)
    for call, m in enumerate(rows):
        print(f"noalloc call {call}: {bits}-bit g{group} d={d} ffn={ffn} m={m}", flush=True)
        x = W.generic_act((61, m, 1), (m, d), "bf16")
        r = W.generic_act((61, m, 2), (m, d), "bf16")
        xd, rd = to_device(x), to_device(r)
        out_na = torch.empty_like(rd)
        assert _call_noalloc(qdm, xd, rd, gu, dn, out_na) == qdm.QDM_OK
        ws = torch.empty(qdm.mlp_workspace_bytes(m, qdm.QDM_BF16, gu, dn), dtype=torch.uint8, device="cuda")
        out_ws = qdm.mlp_decode(xd, rd, gu, dn, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws)
        _, y_ref = oracle.mlp_decode(x.values, r.values, ow.wg, ow.wu, ow.wd)
        err = oracle.scaled_error(from_device(out_na), y_ref)
        print(f"  bitwise equal; error vs oracle {err:.3e}", flush=True)
        assert err <= TOL["bf16"], err


def test_noalloc_refuses_more_than_its_array():
    import quantized_decode_mlp_amd as qdm
    d, ffn = 4096, 14336
    _, (gu, dn) = generic_case((62, 4, 64), d, ffn, 4, 64, sigma=0.02)
    m = 128   # h alone is 7.3 MB, the tiled kernels' partials 29 MB more
    assert qdm.mlp_workspace_bytes(m, qdm.QDM_BF16, gu, dn) > qdm.NOALLOC_SCRATCH_BYTES
    xd = torch.zeros((m, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((m, d), 7.0, dtype=torch.bfloat16, device="cuda")
    assert _call_noalloc(qdm, xd, xd, gu, dn, out) == qdm.QDM_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing ran
