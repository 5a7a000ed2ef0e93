"""Seeded synthetic inputs for the one-row quantized decode MLP.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds shapes, distributions and seeds only: no quantization, no packing,
no dot products, no normalisation.  The one piece of arithmetic it performs
is rounding freshly drawn fp32 activations to the storage dtype of a
workload (bf16 / f16), which is input preparation, so that both sides of a
comparison read the very same bits.

The workloads mirror the MLP shapes of the models the meTile "MLX-LM
Backend" page benchmarks (Llama 3.2 1B, Qwen 2.5 1.5B, Qwen 3 8B, Llama 3
8B).  Those checkpoints are not used: weights are Gaussian with the stated
sigma, activations standard normal.

Seeds: every tensor is drawn from ``numpy.random.default_rng`` seeded with
``SeedSequence([workload_index, set_index, tensor_id])``; tensor ids are
1 W_gate, 2 W_up, 3 W_down, 4 x, 5 r, 6 a, 7 b, 8 norm weight, 9-11 the decode
chain's a, b and norm weight.
Activations are drawn in fp32 as one [M, d] block, so the first row of an
M-row draw equals the 1-row draw.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

TENSOR_IDS = {"w_gate": 1, "w_up": 2, "w_down": 3, "x": 4, "r": 5,
              "a": 6, "b": 7, "norm_w": 8, "chain_a": 9, "chain_b": 10, "chain_w": 11}

DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class Workload:
    index: int            # 1-based workload number
    name: str
    d: int                # model width (input dim of gate/up, output dim of down)
    ffn: int              # hidden width
    bits: int             # 8 = uint8 affine, 4 = two codes per byte, 16 = dense bf16
    group: int            # affine group along the input dim; 0 for dense
    act: str              # activation / residual / output dtype
    sigma: float          # weight standard deviation
    n_sets: int = 1       # independent weight sets (rotated per call)
    rows: Tuple[int, ...] = (1,)
    norm_dtype: Optional[str] = None   # add+RMSNorm dtype, when the workload has one
    norm_eps: float = 1e-5

    @property
    def weight_bytes(self) -> int:
        """Algorithmic weight bytes of one layer: packed codes plus the fp32
        (scale, bias) pair of every group, or the dense bf16 weights."""
        n_w = 3 * self.d * self.ffn
        if self.bits == 16:
            return 2 * n_w
        q = n_w * self.bits // 8
        return q + 8 * (n_w // self.group)


WORKLOADS = {
    1: Workload(1, "tiny d256 ffn512 uint8 g32 fp32", 256, 512, 8, 32, "f32", 0.05,
                norm_dtype="f32"),
    2: Workload(2, "Llama-3.2-1B-shaped d2048 ffn8192 uint8 g64 bf16", 2048, 8192, 8, 64,
                "bf16", 0.02, norm_dtype="f16"),
    3: Workload(3, "Qwen2.5-1.5B-shaped d1536 ffn8960 dense bf16", 1536, 8960, 16, 0,
                "bf16", 0.02),
    4: Workload(4, "Qwen3-8B-shaped d4096 ffn12288 uint8 g128 bf16 x36 layers", 4096,
                12288, 8, 128, "bf16", 0.02, n_sets=36),
    5: Workload(5, "Llama-3-8B-shaped d4096 ffn14336 uint4 g64 bf16 M1/4/16", 4096, 14336,
                4, 64, "bf16", 0.02, rows=(1, 4, 16)),
}


@dataclass(frozen=True)
class Projection:
    """A one-row decode projection other than the MLP (vocabulary or attention)."""
    key: str
    name: str
    n: int                # output rows (vocabulary size, or the projection's width)
    k: int                # input dim
    bits: int
    group: int
    act: str
    sigma: float          # weight standard deviation
    bias: bool            # the projection keeps a bias
    seed_id: int

    @property
    def weight_bytes(self) -> int:
        if self.bits == 16:
            return 2 * self.n * self.k
        return self.n * self.k * self.bits // 8 + 8 * (self.n * self.k // self.group)


# Vocabulary projections at the shapes of the pages' Qwen 3 8B (untied
# lm_head) and Llama 3.2 1B (tied embedding used as the output map), and the
# attention projections of a Qwen 2.5 1.5B-shaped layer (q/k/v with biases, o
# without; 12 query and 2 key/value heads of 128) at affine group 32.
PROJECTIONS = {p.key: p for p in (
    Projection("qwen3_8b_lm_head", "Qwen3-8B-shaped untied lm_head: vocab 151936 x d 4096, uint8 g128",
               151936, 4096, 8, 128, "bf16", 0.02, False, 101),
    Projection("llama32_1b_tied_embedding", "Llama-3.2-1B-shaped tied embedding as output map: vocab 128256 "
               "x d 2048, uint8 g64", 128256, 2048, 8, 64, "bf16", 0.02, False, 102),
    Projection("qwen25_1p5b_q", "Qwen2.5-1.5B-shaped q_proj 1536 x 1536 + bias, uint8 g32",
               1536, 1536, 8, 32, "bf16", 0.02, True, 103),
    Projection("qwen25_1p5b_k", "Qwen2.5-1.5B-shaped k_proj 256 x 1536 + bias, uint8 g32",
               256, 1536, 8, 32, "bf16", 0.02, True, 104),
    Projection("qwen25_1p5b_v", "Qwen2.5-1.5B-shaped v_proj 256 x 1536 + bias, uint8 g32",
               256, 1536, 8, 32, "bf16", 0.02, True, 105),
    Projection("qwen25_1p5b_o", "Qwen2.5-1.5B-shaped o_proj 1536 x 1536, uint8 g32",
               1536, 1536, 8, 32, "bf16", 0.02, False, 106),
)}


def projection_inputs(p: Projection, m: int = 1, copy: int = 0):
    """(W fp32 [n, k] ~ N(0, sigma), bias Act [n] ~ N(0, 0.1) or None, x Act [m, k] ~ N(0, 1))."""
    def rng(t):
        return np.random.default_rng(np.random.SeedSequence([p.seed_id, copy, t]))
    w = normal_f32(rng(1), (p.n, p.k), p.sigma)
    b = to_storage(normal_f32(rng(2), (p.n,), 0.1), p.act) if p.bias else None
    x = to_storage(normal_f32(rng(3), (m, p.k)), p.act)
    return w, b, x


def rng_for(workload: int, set_index: int, tensor: str) -> np.random.Generator:
    seq = np.random.SeedSequence([int(workload), int(set_index), TENSOR_IDS[tensor]])
    return np.random.default_rng(seq)


def normal_f32(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


# ---------------------------------------------------------------- storage dtypes

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Act:
    """A host activation array in its storage dtype.

    ``values`` holds the exact stored values as fp32 (every bf16/f16 value is
    an fp32 value); ``raw`` holds the storage bits (uint16 for bf16/f16,
    the fp32 array itself for f32)."""
    dtype: str
    values: np.ndarray
    raw: np.ndarray


def to_storage(a: np.ndarray, dtype: str) -> Act:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return Act("f32", a, a)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(a)
        return Act("bf16", bf16_bits_to_f32(bits), bits)
    if dtype == "f16":
        h = a.astype(np.float16)
        return Act("f16", h.astype(np.float32), h.view(np.uint16))
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- draws

def weights_f32(w: Workload, set_index: int = 0):
    """fp32 draws of (W_gate [ffn,d], W_up [ffn,d], W_down [d,ffn])."""
    g = normal_f32(rng_for(w.index, set_index, "w_gate"), (w.ffn, w.d), w.sigma)
    u = normal_f32(rng_for(w.index, set_index, "w_up"), (w.ffn, w.d), w.sigma)
    dn = normal_f32(rng_for(w.index, set_index, "w_down"), (w.d, w.ffn), w.sigma)
    return g, u, dn


def weight_f32(w: Workload, which: str, set_index: int = 0) -> np.ndarray:
    shape = (w.d, w.ffn) if which == "w_down" else (w.ffn, w.d)
    return normal_f32(rng_for(w.index, set_index, which), shape, w.sigma)


def activations(w: Workload, m: int = 1, set_index: int = 0):
    """(x, r): [m, d] standard-normal draws stored in the workload's dtype."""
    x = normal_f32(rng_for(w.index, set_index, "x"), (m, w.d))
    r = normal_f32(rng_for(w.index, set_index, "r"), (m, w.d))
    return to_storage(x, w.act), to_storage(r, w.act)


def rmsnorm_inputs(w: Workload, rows: int = 1, set_index: int = 0):
    """(a, b, weight) for add+RMSNorm: a, b ~ N(0,1) [rows, d], weight ~ U(0.5, 1.5) [d]."""
    if w.norm_dtype is None:
        raise ValueError(f"workload {w.index} has no add+RMSNorm part")
    a = normal_f32(rng_for(w.index, set_index, "a"), (rows, w.d))
    b = normal_f32(rng_for(w.index, set_index, "b"), (rows, w.d))
    nw = rng_for(w.index, set_index, "norm_w").uniform(0.5, 1.5, size=w.d).astype(np.float32)
    dt = w.norm_dtype
    return to_storage(a, dt), to_storage(b, dt), to_storage(nw, dt)


def chain_inputs(w: Workload, rows: int = 1, set_index: int = 0):
    """(a, b, weight) for the decode chain (add + RMSNorm feeding the MLP), in
    the MLP's activation dtype: a (the residual stream) and b (the block
    output added to it) ~ N(0,1) [rows, d], weight ~ U(0.5, 1.5) [d] -- the
    add+RMSNorm recipe at the MLP's shape."""
    a = normal_f32(rng_for(w.index, set_index, "chain_a"), (rows, w.d))
    b = normal_f32(rng_for(w.index, set_index, "chain_b"), (rows, w.d))
    nw = rng_for(w.index, set_index, "chain_w").uniform(0.5, 1.5, size=w.d).astype(np.float32)
    return to_storage(a, w.act), to_storage(b, w.act), to_storage(nw, w.act)


def generic_weights(seed, n: int, k: int, sigma: float = 0.02) -> np.ndarray:
    """An fp32 [n, k] Gaussian draw for tests of arbitrary shapes."""
    return normal_f32(np.random.default_rng(np.random.SeedSequence(list(seed))), (n, k), sigma)


def generic_act(seed, shape, dtype: str, sigma: float = 1.0) -> Act:
    a = normal_f32(np.random.default_rng(np.random.SeedSequence(list(seed))), shape, sigma)
    return to_storage(a, dtype)


# ---------------------------------------------------------------- edge-case draws
#
# Structured inputs for the parity cases that stress the kernels' decoding:
# groups whose codes sit at the two ends of the range, constant groups,
# activations of one sign, and activations spanning many binades inside one
# 16-element run.  These only place values; what the quantizer makes of them
# is the quantizer's business.

EDGE_WEIGHTS = ("outlier", "constant", "gaussian")
EDGE_ACTS = ("positive", "wide", "gaussian")


def edge_weights(pattern: str, seed, n: int, k: int, group: int, sigma: float = 0.02) -> np.ndarray:
    """fp32 [n, k] weights by group of ``group`` columns.

    outlier:  every group holds one common value (its minimum, ~ N(0, sigma))
              in all places but one, which lies above it by |N(0, 5 sigma)| + 2.5 sigma;
    constant: every other group is constant (a non-zero ~ N(0, sigma) value,
              pushed away from 0), the others ~ N(0, sigma);
    gaussian: ~ N(0, sigma)."""
    if k % group:
        raise ValueError("k must be a multiple of group")
    rng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    ng = k // group
    if pattern == "gaussian":
        return normal_f32(rng, (n, k), sigma)
    if pattern == "outlier":
        base = normal_f32(rng, (n, ng), sigma)
        w = np.repeat(base[:, :, None], group, axis=2)
        pos = rng.integers(0, group, size=(n, ng))
        lift = (np.abs(normal_f32(rng, (n, ng), 5 * sigma)) + np.float32(2.5 * sigma)).astype(np.float32)
        rows, cols = np.meshgrid(np.arange(n), np.arange(ng), indexing="ij")
        w[rows, cols, pos] = base + lift
        return np.ascontiguousarray(w.reshape(n, k), dtype=np.float32)
    if pattern == "constant":
        w = normal_f32(rng, (n, ng, group), sigma)
        c = normal_f32(rng, (n, ng), sigma)
        c = np.where(np.abs(c) < sigma / 4, np.float32(sigma / 2), c).astype(np.float32)
        w[:, 0::2, :] = c[:, 0::2, None]
        return np.ascontiguousarray(w.reshape(n, k), dtype=np.float32)
    raise ValueError(f"unknown weight pattern {pattern!r}")


def edge_activations(pattern: str, seed, shape, dtype: str) -> Act:
    """Activations [.., d] in ``dtype``.

    positive: |N(0, 1)|;
    wide:     random signs, magnitudes (1 + U[0,1)) * 2^e with e uniform in
              [-14, 2], and in every aligned run of 16 elements the first at
              (1 + U[0,1)) * 2^6 and the second exactly 2^-14, so each run
              spans at least 2^20 (all f16 normals; small enough that an MLP's
              outputs stay inside the f16 range);
    gaussian: N(0, 1)."""
    rng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    if pattern == "gaussian":
        return to_storage(normal_f32(rng, shape), dtype)
    if pattern == "positive":
        return to_storage(np.abs(normal_f32(rng, shape)), dtype)
    if pattern == "wide":
        d = shape[-1]
        if d % 16:
            raise ValueError("the last dim must be a multiple of 16")
        e = rng.integers(-14, 3, size=shape)
        e[..., 0::16] = 6
        mag = (1.0 + rng.random(size=shape)) * np.exp2(e)
        mag[..., 1::16] = 2.0 ** -14
        sign = np.where(rng.random(size=shape) < 0.5, -1.0, 1.0)
        return to_storage((sign * mag).astype(np.float32), dtype)
    raise ValueError(f"unknown activation pattern {pattern!r}")
