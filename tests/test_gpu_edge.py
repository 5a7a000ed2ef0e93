"""GPU parity on structured inputs that stress how the kernels decode codes.

The one-row kernels take 8/4-bit codes as exact f16 values under a fixed
exponent (1024 + c, or 1 + n/16) and remove the offset's share per chunk,
and hold 16-bit activations as f16 after a per-lane power-of-two scale; the
few-row kernels take codes as exact 16-bit matrix operands with a per-group
fp32 fold.  These cases put the codes at the ends of their range (one code at
2^bits - 1 in a group otherwise at its minimum), make groups constant, give
the activations one sign (the offset's share then cancels with no help from
signs), or spread one 16-element run of activations over 2^19 and more.

Bars as everywhere: the fp32 hidden row h within 1e-5 and the 16-bit output
within 5e-3 of the fp64 oracle (max |out - ref| / max |ref|).  Both sides
start from the same fp32 weight draws; each quantizes them itself."""
import functools

import pytest

import oracle
import workloads as W
from gpu_cases import H_TOL, TOL, from_device, oracle_weights_from_f32, product_weights_from_f32, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# d and ffn are multiples of 512 (the few-row kernels' k-block runs) that leave
# ragged last K-tiles in the one-row kernels: 3584 uint8 codes are 3.5 tiles
# of 1 KiB, 2560 are 2.5.
D, FFN = 3584, 2560
FORMATS = [(8, 128), (4, 64), (8, 32)]
CASES = [("outlier", "gaussian"), ("outlier", "positive"), ("gaussian", "wide"), ("constant", "positive"),
         ("outlier", "wide")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a GPU")
    import quantized_decode_mlp_amd  # noqa: F401
    yield
    torch.cuda.synchronize()


@functools.lru_cache(maxsize=None)
def _weights(wpat, bits, group):
    seed = (900 + bits, group, W.EDGE_WEIGHTS.index(wpat))
    g32 = W.edge_weights(wpat, seed + (1,), FFN, D, group)
    u32 = W.edge_weights(wpat, seed + (2,), FFN, D, group)
    d32 = W.edge_weights(wpat, seed + (3,), D, FFN, group)
    return (oracle_weights_from_f32(g32, u32, d32, bits, group),
            product_weights_from_f32(g32, u32, d32, bits, group))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("wpat,xpat", CASES)
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("m", [1, 16])
def test_edge_mlp(bits, group, wpat, xpat, act, m):
    import quantized_decode_mlp_amd as qdm
    ow, (gu, dn) = _weights(wpat, bits, group)
    seed = (950, m, W.EDGE_ACTS.index(xpat), 0 if act == "bf16" else 1)
    x = W.edge_activations(xpat, seed + (4,), (m, D), act)
    r = W.edge_activations("gaussian", seed + (5,), (m, D), act)
    print(f"edge case: {bits}-bit g{group} weights {wpat}, x {xpat} {act}, m={m}", flush=True)
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
