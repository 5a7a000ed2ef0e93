"""Pins for the oracle's packer (CPU): hand-written bytes, round trips and
the gate/up interleave index map."""
import numpy as np
import pytest

import oracle


def test_nibble_bytes_by_hand():
    # low nibble = even k, high nibble = odd k
    codes = np.array([[1, 2, 15, 0, 0, 15, 7, 8]], dtype=np.uint8)
    packed = oracle.pack_codes(codes, 4)
    assert packed.tolist() == [[0x21, 0x0F, 0xF0, 0x87]]


def test_byte_codes_are_identity():
    codes = np.arange(64, dtype=np.uint8).reshape(2, 32) * 3
    assert np.array_equal(oracle.pack_codes(codes, 8), codes)


@pytest.mark.parametrize("bits", [4, 8])
def test_roundtrip(bits):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 1 << bits, size=(5, 96), dtype=np.uint8)
    packed = oracle.pack_codes(codes, bits)
    assert packed.shape == (5, 96 * bits // 8)
    assert np.array_equal(oracle.unpack_codes(packed, bits, 96), codes)


def test_code_out_of_range_rejected():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.array([[16, 0]], dtype=np.uint8), 4)


def test_gate_up_interleave_2x2():
    gate = np.array([[1, 2], [3, 4]], dtype=np.uint8)
    up = np.array([[5, 6], [7, 8]], dtype=np.uint8)
    p = oracle.pack_gate_up(gate, up, 8)
    assert p.shape == (2, 2, 2)
    # packed row 2n = gate row n, 2n+1 = up row n
    assert p.reshape(4, 2).tolist() == [[1, 2], [5, 6], [3, 4], [7, 8]]


def test_scale_bias_layout():
    s = np.array([[1, 2], [3, 4]], dtype=np.float32)
    b = np.array([[-1, -2], [-3, -4]], dtype=np.float32)
    sb = oracle.pack_scale_bias(s, b)
    assert sb.reshape(-1).tolist() == [1, -1, 2, -2, 3, -3, 4, -4]
    s2, b2 = oracle.unpack_scale_bias(sb)
    assert np.array_equal(s2, s) and np.array_equal(b2, b)
    gu = oracle.pack_gate_up_scale_bias(s, b, s * 10, b * 10)
    assert gu.shape == (2, 2, 2, 2)
    assert gu.reshape(-1).tolist() == [1, -1, 2, -2, 10, -10, 20, -20,
                                       3, -3, 4, -4, 30, -30, 40, -40]


def test_dense_interleave():
    g = np.array([[0x3F80, 0x4000]], dtype=np.uint16)
    u = np.array([[0xBF80, 0xC000]], dtype=np.uint16)
    p = oracle.pack_dense_gate_up(g, u)
    assert p.reshape(-1).tolist() == [0x3F80, 0x4000, 0xBF80, 0xC000]
