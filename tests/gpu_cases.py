"""Shared preparation for the GPU parity tests.

Both sides start from the same seeded fp32 draws (``workloads``).  The
oracle quantizes and dequantizes them itself (fp64); the product quantizes
and packs them with the library's host code and uploads the packed bytes.
Nothing the product computes is fed to the oracle."""
from __future__ import annotations

import functools
from dataclasses import dataclass

import numpy as np

import oracle
import workloads as W

TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 5e-3}
H_TOL = 1e-5


@dataclass
class OracleMLP:
    wg: np.ndarray     # fp64 [ffn, d]
    wu: np.ndarray
    wd: np.ndarray     # fp64 [d, ffn]


def oracle_weights_from_f32(g32, u32, d32, bits, group) -> OracleMLP:
    if bits == 16:
        deq = [oracle.dequantize_dense_bf16(W.to_storage(a, "bf16").raw) for a in (g32, u32, d32)]
    else:
        deq = []
        for a in (g32, u32, d32):
            c, s, b = oracle.quantize_affine(a, bits, group)
            deq.append(oracle.dequantize(c, s, b, group))
    return OracleMLP(*deq)


def product_weights_from_f32(g32, u32, d32, bits, group):
    import quantized_decode_mlp_amd as qdm
    ffn, d = g32.shape
    if bits == 16:
        gb = W.to_storage(g32, "bf16").raw
        ub = W.to_storage(u32, "bf16").raw
        db = W.to_storage(d32, "bf16").raw
        gu = qdm.Weight.from_host(ffn, d, 16, 0, qdm.pack_dense_gate_up(gb, ub), None)
        dn = qdm.Weight.from_host(d, ffn, 16, 0, db, None)
    else:
        q, sb = qdm.quantize_pack_gate_up(g32, u32, bits, group)
        gu = qdm.Weight.from_host(ffn, d, bits, group, q, sb)
        dq, dsb = qdm.quantize_pack_rows(d32, bits, group)
        dn = qdm.Weight.from_host(d, ffn, bits, group, dq, dsb)
    return gu, dn


@functools.lru_cache(maxsize=4)
def workload_case(index: int, set_index: int = 0):
    """(oracle weights, product weights) for a workload's weight set."""
    wl = W.WORKLOADS[index]
    g32, u32, d32 = W.weights_f32(wl, set_index)
    ow = oracle_weights_from_f32(g32, u32, d32, wl.bits, wl.group)
    pw = product_weights_from_f32(g32, u32, d32, wl.bits, wl.group)
    return ow, pw


def generic_case(seed, d, ffn, bits, group, sigma=0.05):
    g32 = W.generic_weights((seed, 1), ffn, d, sigma)
    u32 = W.generic_weights((seed, 2), ffn, d, sigma)
    d32 = W.generic_weights((seed, 3), d, ffn, sigma)
    return (oracle_weights_from_f32(g32, u32, d32, bits, group),
            product_weights_from_f32(g32, u32, d32, bits, group))


def to_device(act: W.Act):
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[act.dtype]
    raw = np.ascontiguousarray(act.raw)
    t = torch.from_numpy(raw) if act.dtype == "f32" else torch.from_numpy(raw.view(np.int16)).view(tdt)
    return t.to("cuda")


def from_device(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
