"""Host quantize/pack (C++, in libqdm.so) against the oracle (CPU): byte for
byte, on every workload's shapes and on fuzzed shapes, values and ties."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import quantized_decode_mlp_amd as q
import workloads as W


def _oracle_rows(w, bits, group):
    c, s, b = oracle.quantize_affine(w, bits, group)
    return c, s, b, oracle.pack_codes(c, bits), oracle.pack_scale_bias(s, b)


def _assert_same_f32(a, b):
    assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@pytest.mark.parametrize("wl,rows", [(1, None), (2, None), (4, 192), (5, 160)])
def test_workload_shapes_bit_exact(wl, rows):
    w = W.WORKLOADS[wl]
    for which in ("w_gate", "w_down"):
        full = W.weight_f32(w, which)
        m = full if rows is None else full[:rows]
        c, s, b, qp, sbp = _oracle_rows(m, w.bits, w.group)
        c2, s2, b2 = q.quantize_affine(m, w.bits, w.group)
        assert np.array_equal(c, c2)
        _assert_same_f32(s, s2)
        _assert_same_f32(b, b2)
        qp2, sbp2 = q.quantize_pack_rows(m, w.bits, w.group)
        assert np.array_equal(qp, qp2)
        _assert_same_f32(sbp, sbp2)
        qp3, sbp3 = q.pack_rows(c, s, b, w.bits, w.group)
        assert np.array_equal(qp, qp3)
        _assert_same_f32(sbp, sbp3)


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 128), (4, 32)])
def test_gate_up_interleave_bit_exact(bits, group):
    wg = W.generic_weights((1, bits), 48, 256, 0.02)
    wu = W.generic_weights((2, bits), 48, 256, 0.02)
    gc, gs, gb = oracle.quantize_affine(wg, bits, group)
    uc, us, ub = oracle.quantize_affine(wu, bits, group)
    qo = oracle.pack_gate_up(gc, uc, bits)
    sbo = oracle.pack_gate_up_scale_bias(gs, gb, us, ub)
    q1, sb1 = q.quantize_pack_gate_up(wg, wu, bits, group)
    assert np.array_equal(qo, q1)
    _assert_same_f32(sbo, sb1)
    q2, sb2 = q.pack_gate_up(gc, gs, gb, uc, us, ub, bits, group)
    assert np.array_equal(qo, q2)
    _assert_same_f32(sbo, sb2)


def test_dense_interleave_bit_exact():
    rng = np.random.default_rng(0)
    g = rng.integers(0, 1 << 16, size=(40, 24), dtype=np.uint16)
    u = rng.integers(0, 1 << 16, size=(40, 24), dtype=np.uint16)
    assert np.array_equal(q.pack_dense_gate_up(g, u), oracle.pack_dense_gate_up(g, u))


def test_hand_golden_groups():
    """The hand-built ties and rounded-scale cases, through the C++ quantizer."""
    from conftest import load_golden
    for case in load_golden("quantize_hand.json")["cases"]:
        if "multipliers" in case:
            w = (case["min"] + case["step"] * np.asarray(case["multipliers"])).astype(np.float32)
        elif "values" in case:
            w = np.asarray(case["values"], np.float32)
        else:
            w = np.full(32, case["constant"], np.float32)
        c, s, b = q.quantize_affine(w[None, :], case["bits"], case["group"])
        if "codes" in case:
            assert c[0].tolist() == case["codes"]
        assert float(s[0, 0]) == case["scale"]


def test_signed_zero_minimum():
    w = np.zeros((2, 32), np.float32)
    w[0, 5] = -0.0
    w[0, 7] = 1.0
    w[1, :] = -0.0
    c, s, b = q.quantize_affine(w, 8, 32)
    c2, s2, b2 = oracle.quantize_affine(w, 8, 32)
    _assert_same_f32(b, b2)
    assert np.all(np.signbit(b) == False)  # noqa: E712


_groups = st.sampled_from([32, 64, 128])


@settings(max_examples=60, deadline=None)
@given(bits=st.sampled_from([4, 8]), group=_groups, n=st.integers(1, 9), ng=st.integers(1, 4),
       seed=st.integers(0, 2 ** 31 - 1), mode=st.sampled_from(["normal", "grid", "wide", "const"]))
def test_fuzz_bit_exact(bits, group, n, ng, seed, mode):
    rng = np.random.default_rng(seed)
    k = group * ng
    if mode == "normal":
        w = rng.standard_normal((n, k)).astype(np.float32) * np.float32(rng.uniform(1e-3, 10))
    elif mode == "grid":
        # values on an exact grid with half steps: exercises ties
        step = np.float32(2.0 ** rng.integers(-12, 2))
        mult = rng.integers(0, 2 * ((1 << bits) - 1) + 1, size=(n, k)) / 2.0
        mult[:, 0] = 0
        mult[:, 1] = (1 << bits) - 1
        w = (np.float32(rng.uniform(-4, 4)) + step * mult).astype(np.float32)
    elif mode == "wide":
        w = (rng.standard_normal((n, k)) * np.exp(rng.uniform(-30, 30, (n, k)))).astype(np.float32)
    else:
        w = np.full((n, k), np.float32(rng.standard_normal()), np.float32)
        w[:, ::7] = np.float32(rng.standard_normal())
    c, s, b, qp, sbp = _oracle_rows(w, bits, group)
    qp2, sbp2 = q.quantize_pack_rows(w, bits, group)
    assert np.array_equal(qp, qp2)
    _assert_same_f32(sbp, sbp2)
    c2, s2, b2 = q.quantize_affine(w, bits, group)
    assert np.array_equal(c, c2)


# ------------------------------------------------------------------ MX block-scaled

MX = [(q.QDM_MXFP4, "mxfp4"), (q.QDM_MXFP8, "mxfp8")]


@pytest.mark.parametrize("fmt,name", MX)
def test_mx_workload_shapes_bit_exact(fmt, name):
    for wl, rows in ((4, 128), (5, 96), (2, 128)):
        w = W.weight_f32(W.WORKLOADS[wl], "w_gate")[:rows]
        c, e = oracle.quantize_mx(w, name)
        q1, e1 = q.quantize_mx(w, fmt)
        assert np.array_equal(q1, oracle.pack_mx_codes(c, name))
        assert np.array_equal(e1, e)


@pytest.mark.parametrize("fmt,name", MX)
def test_mx_edge_values_bit_exact(fmt, name):
    rng = np.random.default_rng(11)
    w = rng.normal(size=(8, 128)).astype(np.float32)
    w[0, :32] = 0.0                                   # zero block
    w[1, :32] = -0.0
    w[1, 32:64] = np.float32(1e-42)                   # subnormal fp32 inputs
    w[2, :32] = np.float32(3.0e38)                    # near the fp32 maximum
    w[2, 32:64] = rng.normal(size=32).astype(np.float32) * np.float32(2.0 ** -130)
    w[3, :32] = np.tile(np.array([6.0, 2.5, 3.5, 5.0, -0.2, 0.25, 0.75, 7.5], np.float32), 4)
    w[4] = np.round(w[4] * 8) / 8                     # many ties
    c, e = oracle.quantize_mx(w, name)
    q1, e1 = q.quantize_mx(w, fmt)
    assert np.array_equal(q1, oracle.pack_mx_codes(c, name))
    assert np.array_equal(e1, e)


@pytest.mark.parametrize("fmt,name", MX)
def test_mx_gate_up_interleave(fmt, name):
    wg = W.generic_weights((3, fmt), 24, 256, 0.02)
    wu = W.generic_weights((4, fmt), 24, 256, 0.02)
    q1, e1 = q.quantize_mx_gate_up(wg, wu, fmt)
    for v, w in enumerate((wg, wu)):
        c, e = oracle.quantize_mx(w, name)
        assert np.array_equal(q1[:, v], oracle.pack_mx_codes(c, name))
        assert np.array_equal(e1[:, v], e)


def test_mx_rejects():
    w = np.zeros((2, 64), np.float32)
    L = q._lib
    qb, eb = np.empty(128, np.uint8), np.empty(4, np.uint8)
    assert L.qdm_quantize_mx(q._ptr(w), 2, 64, 0x105, q._ptr(qb), q._ptr(eb)) == q.QDM_ERR_UNSUPPORTED
    assert L.qdm_quantize_mx(q._ptr(w), 2, 48, q.QDM_MXFP8, q._ptr(qb), q._ptr(eb)) == q.QDM_ERR_INVALID_ARG
    w[1, 3] = np.nan
    assert L.qdm_quantize_mx(q._ptr(w), 2, 64, q.QDM_MXFP8, q._ptr(qb), q._ptr(eb)) == q.QDM_ERR_INVALID_ARG
    assert q.mx_scale_bytes(4096, 12288) == 4096 * 384
    assert q.mx_scale_bytes(4, 48) == 0
    assert q.packed_q_bytes(4, 64, q.QDM_MXFP4) == 128 and q.packed_q_bytes(4, 64, q.QDM_MXFP8) == 256


# ------------------------------------------------------------------ affine with bf16 (scale, bias)

def _bf16_bits(v):
    return (np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32), (8, 128), (4, 64), (8, 32), (4, 128)])
def test_sb16_bit_exact(bits, group):
    for wl, rows in ((4, 96), (5, 64)):
        w = W.weight_f32(W.WORKLOADS[wl], "w_down")[:rows]
        c, s, b = oracle.quantize_affine_bf16sb(w, bits, group)
        q1, sb1 = q.quantize_pack_rows_sb16(w, bits, group)
        assert np.array_equal(q1, oracle.pack_codes(c, bits))
        assert np.array_equal(sb1[..., 0], _bf16_bits(s)) and np.array_equal(sb1[..., 1], _bf16_bits(b))


def test_sb16_gate_up_interleave():
    wg = W.generic_weights((5, 1), 40, 256, 0.02)
    wu = W.generic_weights((5, 2), 40, 256, 0.02)
    q1, sb1 = q.quantize_pack_gate_up_sb16(wg, wu, 4, 64)
    for v, w in enumerate((wg, wu)):
        c, s, b = oracle.quantize_affine_bf16sb(w, 4, 64)
        assert np.array_equal(q1[:, v], oracle.pack_codes(c, 4))
        assert np.array_equal(sb1[:, v, :, 0], _bf16_bits(s)) and np.array_equal(sb1[:, v, :, 1], _bf16_bits(b))


def test_sb16_rejects():
    L = q._lib
    w = np.zeros((2, 64), np.float32)
    qb, sb = np.empty(128, np.uint8), np.empty(16, np.uint16)
    assert L.qdm_quantize_pack_rows_sb16(q._ptr(w), 2, 64, 6, 32, q._ptr(qb), q._ptr(sb)) == q.QDM_ERR_UNSUPPORTED
    assert L.qdm_quantize_pack_rows_sb16(q._ptr(w), 2, 64, 8, 48, q._ptr(qb), q._ptr(sb)) == q.QDM_ERR_UNSUPPORTED
    w[0, 1] = np.inf
    assert L.qdm_quantize_pack_rows_sb16(q._ptr(w), 2, 64, 8, 32, q._ptr(qb), q._ptr(sb)) == q.QDM_ERR_INVALID_ARG
    assert q.packed_q_bytes(4, 64, q.QDM_U4_SB16) == 128 and q.packed_q_bytes(4, 64, q.QDM_U8_SB16) == 256


@pytest.mark.parametrize("bits,group", [(8, 32), (4, 64)])
def test_stacked_rows_pack_as_concatenation(bits, group):
    """Rows are quantized one by one, so the packing of stacked matrices (a
    fused q/k/v weight) is the concatenation of their packings, bytes and
    (scale, bias) pairs alike."""
    mats = [W.generic_weights((bits, group, i), n, 256, 0.02) for i, n in enumerate((48, 16, 16))]
    parts = [q.quantize_pack_rows(a, bits, group) for a in mats]
    codes, sb = q.quantize_pack_rows(np.concatenate(mats), bits, group)
    assert np.array_equal(codes, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(sb, np.concatenate([p[1] for p in parts]))
