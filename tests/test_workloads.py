"""The seeded input generators (CPU): determinism, shapes, storage rounding."""
import numpy as np
import torch

import workloads as W


def test_weight_bytes_table():
    assert W.WORKLOADS[1].weight_bytes == 491_520
    assert W.WORKLOADS[2].weight_bytes == 56_623_104
    assert W.WORKLOADS[3].weight_bytes == 82_575_360
    assert W.WORKLOADS[4].weight_bytes == 160_432_128
    assert W.WORKLOADS[5].weight_bytes == 110_100_480


def test_deterministic_and_distinct():
    w = W.WORKLOADS[1]
    g1, u1, d1 = W.weights_f32(w, 0)
    g2, u2, d2 = W.weights_f32(w, 0)
    assert np.array_equal(g1, g2) and np.array_equal(d1, d2)
    assert g1.shape == (512, 256) and d1.shape == (256, 512)
    assert not np.array_equal(g1, u1)
    g3, _, _ = W.weights_f32(w, 1)
    assert not np.array_equal(g1, g3)
    assert abs(float(g1.std()) - 0.05) < 0.002


def test_first_row_of_multirow_draw():
    w = W.WORKLOADS[1]
    x1, r1 = W.activations(w, 1)
    x4, r4 = W.activations(w, 4)
    assert np.array_equal(x1.values[0], x4.values[0])


def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 7
    act = W.to_storage(a, "bf16")
    t = torch.from_numpy(a).to(torch.bfloat16)
    assert np.array_equal(act.raw, t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(act.values, t.float().numpy())


def test_f16_storage():
    a = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    act = W.to_storage(a, "f16")
    assert act.raw.dtype == np.uint16
    assert np.array_equal(act.values, a.astype(np.float16).astype(np.float32))


def test_rmsnorm_inputs():
    a, b, nw = W.rmsnorm_inputs(W.WORKLOADS[2])
    assert a.dtype == "f16" and a.values.shape == (1, 2048)
    assert nw.values.min() >= 0.5 and nw.values.max() <= 1.5


def test_chain_inputs():
    for i in (1, 2, 3, 4, 5):
        wl = W.WORKLOADS[i]
        a, b, nw = W.chain_inputs(wl, 2)
        assert a.dtype == b.dtype == nw.dtype == wl.act
        assert a.values.shape == b.values.shape == (2, wl.d) and nw.values.shape == (wl.d,)
        assert nw.values.min() >= 0.5 and nw.values.max() <= 1.5
        assert not np.array_equal(a.values, b.values)
    a1, _, _ = W.chain_inputs(W.WORKLOADS[4], 1)
    a2, _, _ = W.chain_inputs(W.WORKLOADS[4], 2)
    assert np.array_equal(a1.values[0], a2.values[0])


def test_projection_inputs():
    for key, p in W.PROJECTIONS.items():
        if p.n * p.k > 10_000_000:
            continue
        w, b, x = W.projection_inputs(p, 3)
        assert w.shape == (p.n, p.k) and x.values.shape == (3, p.k) and x.dtype == p.act
        assert (b is not None) == p.bias
        w2, _, _ = W.projection_inputs(p, 1)
        assert np.array_equal(w, w2)
    assert W.PROJECTIONS["qwen3_8b_lm_head"].weight_bytes == 151936 * 4096 + 8 * 151936 * 4096 // 128
