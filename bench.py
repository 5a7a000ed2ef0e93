"""Benchmark of the one-row quantized decode MLP on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME[,NAME...]]

Headline workload: the Qwen3-8B-shaped MLP stack -- d = 4096, ffn = 12288,
affine uint8 weights with groups of 128 along the input dim, 36 independent
layer weight sets (5.78 GB, far beyond the 256 MB Infinity Cache and the
L2s) resident in HBM and rotated per call, 1 activation row in bf16.  One
step = one MLP layer decode (the gate/up + SwiGLU kernel and the down +
residual kernel) on layer (step mod 36).

Timed region: W eager warm-up steps and --warmup-ms of untimed graph
replays, then whole replays of a HIP graph that holds one 36-layer rotation, at least --min-rotations of them and enough to
cover K steps; the steps actually timed are reported (`steps_timed`).  The
time per layer is the HIP-event time of those replays on the launch stream
divided by the layers they ran; the wall-clock time of the same region,
bracketed by device synchronizations, is reported beside it, and the
p10 / p50 / p90 of the region's per-rotation times (events between the
replays).

Every configuration (the headline stack, the decode chain, the other four
workloads, the add + RMSNorm rows, the projections, the group, scale/bias and
MX variants, a launch floor) is captured once as a graph of one rotation over
address-distinct weight copies of at least 2 GiB, and sampled in rounds: each
round replays every configuration once, in an order rotated from round to
round, so drift over the run falls on all of them alike.  Each configuration
reports the p10 / p50 / p90 of its per-layer times over the rounds.

Prints one JSON line: metric, value (weight-stream GB/s = algorithmic weight
bytes per layer / time per layer), the fraction of the 8 TB/s HBM peak, a
roofline record for the dominant kernel (gate/up), the fp64 CPU oracle timed
on a bounded sample on the host cores, and the other configurations.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "µs/MLP layer + weight-stream GB/s (% of 8 TB/s HBM), 1-row decode"
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK = 2.5e15
ACT_CODE = {"f32": 0, "f16": 1, "bf16": 2}   # qdm_dtype of a storage dtype
COPY_BYTES = 2 << 30                          # weight copies per configuration: at least this many bytes


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pcts(v):
    return {"p10": round(float(np.percentile(v, 10)), 3), "p50": round(float(np.percentile(v, 50)), 3),
            "p90": round(float(np.percentile(v, 90)), 3)}


def _copies(nbytes):
    return int(-(-COPY_BYTES // nbytes))


def _dev(a):
    import torch
    if a.dtype == "f32":
        return torch.from_numpy(a.raw).cuda()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[a.dtype]
    return torch.from_numpy(np.ascontiguousarray(a.raw).view(np.int16)).view(tdt).cuda()


class Case:
    """One configuration: `run(i)` enqueues call i of a rotation of n calls; the
    rotation is captured once as a HIP graph and sampled by replaying it."""

    def __init__(self, name, run, n, keep=(), weight_bytes=None, flops=None, info=None):
        import torch
        self.name, self.n, self.keep = name, n, keep
        self.weight_bytes, self.flops, self.info = weight_bytes, flops, dict(info or {})
        for i in range(n):   # eager pass: checks the calls, warms the code objects
            run(i)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(n):
                run(i)
        self.graph.replay()
        torch.cuda.synchronize()
        self.samples = []

    def sample(self):
        import torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        self.graph.replay()
        b.record()
        b.synchronize()
        self.samples.append(a.elapsed_time(b) / self.n * 1e3)

    def record(self):
        med = float(np.median(self.samples))
        key = "us_per_layer" if self.weight_bytes is not None or self.flops is not None else "us"
        rec = {key: pcts(self.samples)}
        if self.weight_bytes is not None:
            gbps = self.weight_bytes / (med * 1e-6) / 1e9
            rec.update(weight_bytes=int(self.weight_bytes), weight_GBps=round(gbps, 1),
                       hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))
        if self.flops is not None:
            rec.update(tflops=round(self.flops / (med * 1e-6) / 1e12, 2),
                       mfma_util_bf16=round(self.flops / (med * 1e-6) / BF16_DENSE_PEAK, 5))
        rec.update(self.info)
        return rec


# ------------------------------------------------------------------ weights

def prepare_sets(wl: W.Workload, n_sets: int):
    """Draws, quantizes and packs n_sets independent weight sets on host threads and uploads them."""
    import torch
    import quantized_decode_mlp_amd as qdm

    def one(s):
        g32, u32, d32 = W.weights_f32(wl, s)
        q, sb = qdm.quantize_pack_gate_up(g32, u32, wl.bits, wl.group)
        dq, dsb = qdm.quantize_pack_rows(d32, wl.bits, wl.group)
        return s, q, sb, dq, dsb

    sets = [None] * n_sets
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=4) as ex:
        for s, q, sb, dq, dsb in ex.map(one, range(n_sets)):
            sets[s] = (qdm.Weight.from_host(wl.ffn, wl.d, wl.bits, wl.group, q, sb),
                       qdm.Weight.from_host(wl.d, wl.ffn, wl.bits, wl.group, dq, dsb))
            if (s + 1) % 6 == 0 or s + 1 == n_sets:
                _log(f"prepared {s + 1}/{n_sets} layer sets ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    return sets


def packed_copies(wl: W.Workload, fmt=None, group=None, copies=None):
    """Copies of set 0 of a workload in a weight format: affine at the workload's
    bits (or `group`), its bf16-pair form ('sb16'), MX ('mxfp8' / 'mxfp4'), or
    dense bf16.  Returns (copies list of (gate_up, down), weight bytes per layer)."""
    import quantized_decode_mlp_amd as qdm
    g32, u32, d32 = W.weights_f32(wl, 0)
    group = group or wl.group
    if wl.bits == 16:
        gb, ub, db = (W.to_storage(a, "bf16").raw for a in (g32, u32, d32))
        q, sb, dq, dsb, bits, es, des = qdm.pack_dense_gate_up(gb, ub), None, db, None, 16, None, None
        grp = 0
    elif fmt in ("mxfp8", "mxfp4"):
        bits = qdm.QDM_MXFP8 if fmt == "mxfp8" else qdm.QDM_MXFP4
        q, es = qdm.quantize_mx_gate_up(g32, u32, bits)
        dq, des = qdm.quantize_mx(d32, bits)
        sb = dsb = None
        grp = 32
    elif fmt == "sb16":
        bits = qdm.QDM_U8_SB16 if wl.bits == 8 else qdm.QDM_U4_SB16
        q, sb = qdm.quantize_pack_gate_up_sb16(g32, u32, wl.bits, group)
        dq, dsb = qdm.quantize_pack_rows_sb16(d32, wl.bits, group)
        es = des = None
        grp = group
    else:
        bits = wl.bits
        q, sb = qdm.quantize_pack_gate_up(g32, u32, wl.bits, group)
        dq, dsb = qdm.quantize_pack_rows(d32, wl.bits, group)
        es = des = None
        grp = group
    del g32, u32, d32
    nbytes = sum(a.nbytes for a in (q, sb, dq, dsb, es, des) if a is not None)
    n = copies or _copies(nbytes)
    sets = [(qdm.Weight.from_host(wl.ffn, wl.d, bits, grp, q, sb, block_scales=es),
             qdm.Weight.from_host(wl.d, wl.ffn, bits, grp, dq, dsb, block_scales=des)) for _ in range(n)]
    return sets, nbytes


def mlp_case(name, wl, sets, nbytes, m, chain=False, info=None):
    """The MLP (or the decode chain) at m rows over the given weight copies."""
    import torch
    import quantized_decode_mlp_amd as qdm
    act = ACT_CODE[wl.act]
    x, r = W.activations(wl, m)
    xd, rd = _dev(x), _dev(r)
    out = torch.empty_like(rd)
    if chain:
        a, b, nw = W.chain_inputs(wl, m)
        ad, bd, nwd = _dev(a), _dev(b), _dev(nw)
        so = torch.empty_like(ad)
        ws = torch.empty(qdm.mlp_rmsnorm_workspace_bytes(m, act, *sets[0]), dtype=torch.uint8, device="cuda")

        def run(i):
            qdm.mlp_decode_rmsnorm(ad, bd, nwd, wl.norm_eps, *sets[i], workspace=ws, s_out=so, out=out)
        keep = (ad, bd, nwd, so, ws, out)
    else:
        ws = torch.empty(qdm.mlp_workspace_bytes(m, act, *sets[0]), dtype=torch.uint8, device="cuda")

        def run(i):
            qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out)
        keep = (xd, rd, ws, out)
    flops = 2 * m * 3 * wl.d * wl.ffn if m > 1 else None
    info = dict(info or {})
    info.setdefault("copies", len(sets))
    return Case(name, run, len(sets), keep=keep + (sets,), weight_bytes=nbytes, flops=flops, info=info)


# ------------------------------------------------------------------ configurations

def headline_cases(sets, wl):
    """The Qwen3-8B-shaped stack (one rotation of its 36 sets), and the decode
    chain on the same sets: add + RMSNorm then the MLP (three launches) and the
    chained call (two launches)."""
    import torch
    import quantized_decode_mlp_amd as qdm
    cases = [mlp_case("headline", wl, sets, wl.weight_bytes, 1, info={"layer_sets": len(sets)})]
    a, b, nw = W.chain_inputs(wl, 1)
    ad, bd, nwd = _dev(a), _dev(b), _dev(nw)
    so, no, out = torch.empty_like(ad), torch.empty_like(ad), torch.empty_like(ad)
    ws = torch.empty(qdm.mlp_workspace_bytes(1, qdm.QDM_BF16, *sets[0]), dtype=torch.uint8, device="cuda")

    def sep(i):
        qdm.add_rmsnorm(ad, bd, nwd, wl.norm_eps, s_out=so, n_out=no)
        qdm.mlp_decode(no, so, *sets[i], workspace=ws, out=out)

    cases.append(Case("decode_chain/add_rmsnorm_then_mlp", sep, len(sets), keep=(ad, bd, nwd, so, no, out, ws),
                      weight_bytes=wl.weight_bytes, info={"launches": 3}))
    c = mlp_case("decode_chain/chained", wl, sets, wl.weight_bytes, 1, chain=True, info={"launches": 2})
    cases.append(c)
    return cases


def _everything(name):
    return True


def workload_cases(want=_everything):
    """Workloads 1, 2, 3 and 5 (5 at 1, 4, 16 rows and at 128 and 512 rows on
    the tiled kernels), the add + RMSNorm rows of workloads 1 and 2 and of the
    Qwen3-8B decode chain (only
    the configurations `want` accepts)."""
    import torch
    import quantized_decode_mlp_amd as qdm
    cases = []
    # workload 1: 0.49 MB of weights stay cache-resident; launch-bound by design
    if want("workload1_m1"):
        wl = W.WORKLOADS[1]
        sets, nbytes = packed_copies(wl, copies=36)
        cases.append(mlp_case("workload1_m1", wl, sets, nbytes, 1,
                              info={"copies": 36, "note": "0.49 MB of weights: cache-resident, launch-bound"}))
    for wi in (1, 2, 4):
        # workload 4 has no standalone add + RMSNorm: its decode chain's norm
        # (the MLP's bf16 activations, d = 4096) stands in
        wl = W.WORKLOADS[wi]
        name = f"add_rmsnorm_{wl.norm_dtype or wl.act}_{wl.d}"
        if not want(name):
            continue
        a, b, w = W.rmsnorm_inputs(wl) if wl.norm_dtype else W.chain_inputs(wl)
        ad, bd, wd = _dev(a), _dev(b), _dev(w)
        so, no = torch.empty_like(ad), torch.empty_like(ad)
        cases.append(Case(name, lambda i: qdm.add_rmsnorm(ad, bd, wd, wl.norm_eps, s_out=so, n_out=no), 36,
                          keep=(ad, bd, wd, so, no)))
    for wi in (2, 3, 5):
        wl = W.WORKLOADS[wi]
        rows = [m for m in (wl.rows + (128, 512) if wi == 5 else (1,)) if want(f"workload{wi}_m{m}")]
        if not rows:
            continue
        sets, nbytes = packed_copies(wl)
        for m in rows:
            cases.append(mlp_case(f"workload{wi}_m{m}", wl, sets, nbytes, m))
            _log(f"captured workload {wi} m={m}")
    if want("launch_floor_fill_kernel"):
        z = torch.empty(1, device="cuda")
        cases.append(Case("launch_floor_fill_kernel", lambda i: z.zero_(), 36, keep=(z,)))
    return cases


def variant_cases(want=_everything):
    """The one-row MLP of each quantized shape at groups 32/64/128; the affine
    formats with bf16 (scale, bias) pairs; MXFP8 / MXFP4 weights."""
    cases = []
    for wi in (2, 4, 5):
        wl = W.WORKLOADS[wi]
        for group in (32, 64, 128):
            name = f"group_sweep/workload{wi}_m1/g{group}"
            if want(name):
                sets, nbytes = packed_copies(wl, group=group)
                cases.append(mlp_case(name, wl, sets, nbytes, 1))
        rows = [m for m in ((1, 4, 16) if wi == 5 else (1,)) if want(f"bf16_scale_bias/workload{wi}_m{m}")]
        if rows:
            sets, nbytes = packed_copies(wl, fmt="sb16")
            for m in rows:
                cases.append(mlp_case(f"bf16_scale_bias/workload{wi}_m{m}", wl, sets, nbytes, m))
        _log(f"captured variants of workload {wi}")
    wl = W.WORKLOADS[4]
    for fmt in ("mxfp8", "mxfp4"):
        if want(f"qwen3_8b_{fmt}_m1"):
            sets, nbytes = packed_copies(wl, fmt=fmt)
            cases.append(mlp_case(f"qwen3_8b_{fmt}_m1", wl, sets, nbytes, 1))
    wl = W.WORKLOADS[5]
    rows = [m for m in wl.rows if want(f"llama3_8b_mxfp4_m{m}")]
    if rows:
        sets, nbytes = packed_copies(wl, fmt="mxfp4")
        for m in rows:
            cases.append(mlp_case(f"llama3_8b_mxfp4_m{m}", wl, sets, nbytes, m))
    return cases


def projection_cases(want=_everything):
    """One-row projections other than the MLP: the Qwen3-8B-shaped lm_head (vocab
    151936), and the attention projections of a Qwen2.5-1.5B-shaped layer (q/k/v
    with bias, o without) in four launches and with q/k/v stacked in two."""
    import torch
    import quantized_decode_mlp_amd as qdm
    cases = []
    if not (want("lm_head_qwen3_8b") or want("attention_qkvo_qwen25_1p5b")
            or want("attention_fused_qkv_o_qwen25_1p5b")):
        return cases

    def prepared(p):
        w32, b, x = W.projection_inputs(p, 1)
        q, sb = qdm.quantize_pack_rows(w32, p.bits, p.group)
        return q, sb, (None if b is None else _dev(b)), _dev(x)

    p = W.PROJECTIONS["qwen3_8b_lm_head"]
    q, sb, _, xd = prepared(p)
    n = _copies(p.weight_bytes)
    ws = [qdm.Weight.from_host(p.n, p.k, p.bits, p.group, q, sb) for _ in range(n)]
    out = torch.empty((1, p.n), dtype=xd.dtype, device="cuda")
    cases.append(Case("lm_head_qwen3_8b", lambda i: qdm.gemv_linear(xd, ws[i], out=out), n, keep=(ws, xd, out),
                      weight_bytes=p.weight_bytes, info={"copies": n}))

    keys = ("qwen25_1p5b_q", "qwen25_1p5b_k", "qwen25_1p5b_v", "qwen25_1p5b_o")
    prep = [prepared(W.PROJECTIONS[k]) for k in keys]
    layer_bytes = sum(W.PROJECTIONS[k].weight_bytes for k in keys)
    n = _copies(layer_bytes)
    layers = [[(qdm.Weight.from_host(W.PROJECTIONS[k].n, W.PROJECTIONS[k].k, W.PROJECTIONS[k].bits,
                                     W.PROJECTIONS[k].group, q, sb), bd)
               for k, (q, sb, bd, _) in zip(keys, prep)] for _ in range(n)]
    xa = prep[0][3]
    outs = [torch.empty((1, W.PROJECTIONS[k].n), dtype=xa.dtype, device="cuda") for k in keys]

    def attn(i):
        for (wt, bd), o in zip(layers[i], outs):
            qdm.gemv_linear(xa, wt, bias=bd, out=o)

    cases.append(Case("attention_qkvo_qwen25_1p5b", attn, n, keep=(layers, xa, outs), weight_bytes=layer_bytes,
                      info={"launches": 4, "copies": n}))
    # q, k and v as one weight (packed rows and their pairs concatenated: every
    # row is quantized on its own) and o: two launches
    n_qkv = sum(W.PROJECTIONS[k].n for k in keys[:3])
    qkv_q = np.ascontiguousarray(np.concatenate([prep[j][0] for j in range(3)], axis=0))
    qkv_sb = np.ascontiguousarray(np.concatenate([prep[j][1] for j in range(3)], axis=0))
    qkv_b = torch.cat([prep[j][2] for j in range(3)])
    po = W.PROJECTIONS[keys[3]]
    fused = [(qdm.Weight.from_host(n_qkv, po.k, po.bits, po.group, qkv_q, qkv_sb),
              qdm.Weight.from_host(po.n, po.k, po.bits, po.group, prep[3][0], prep[3][1])) for _ in range(n)]
    o_qkv = torch.empty((1, n_qkv), dtype=xa.dtype, device="cuda")

    def attn_fused(i):
        qdm.gemv_linear(xa, fused[i][0], bias=qkv_b, out=o_qkv)
        qdm.gemv_linear(xa, fused[i][1], bias=prep[3][2], out=outs[3])

    cases.append(Case("attention_fused_qkv_o_qwen25_1p5b", attn_fused, n, keep=(fused, qkv_b, o_qkv),
                      weight_bytes=layer_bytes, info={"launches": 2, "copies": n}))
    return cases


def sample_interleaved(cases, rounds):
    """`rounds` samples of every case; round r replays the cases starting at
    case r (mod their count), so each case meets every position in the order."""
    n = len(cases)
    for r in range(rounds):
        for j in range(n):
            cases[(r + j) % n].sample()
        if (r + 1) % 5 == 0 or r + 1 == rounds:
            _log(f"sampling round {r + 1}/{rounds} done")


# ------------------------------------------------------------------ dominant kernel

def kernel_event_times(launch, n_layers, launches):
    """Average device duration of one kernel: a HIP graph of n_layers back-to-back
    launches (rotating over the layer sets) is replayed between two HIP events
    recorded on the stream the kernels run on (torch's current stream); the
    elapsed time over the launches."""
    import torch
    for i in range(n_layers):
        launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_layers):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, launches // n_layers)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * n_layers) * 1e3


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qwen3_8b_uint8_g128_mlp_hbm_counters.md")
KERNEL_SOURCES = ["quantized_decode_mlp_amd/csrc/qdm_gemv.hip", "quantized_decode_mlp_amd/csrc/qdm_stream.h",
                  "quantized_decode_mlp_amd/csrc/qdm_device.h", "quantized_decode_mlp_amd/csrc/qdm_launch.h"]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by a plain copy's reading), or None when the kernel
    sources have changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and line[0].isalpha())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    try:
        return int(float(fields["gate_up_traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl: W.Workload, layers: int):
    """The fp64 oracle (as it stands) on `layers` of the workload's layer sets, one
    1-row decode each: dequantize the layer's codes, both projections, SwiGLU,
    residual; the median over the layers.  The oracle's own quantization of
    those layers is setup, not timed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    x, r = W.activations(wl, 1)
    times = []
    for s in range(layers):
        g32, u32, d32 = W.weights_f32(wl, s)
        logical = [oracle.quantize_affine(a, wl.bits, wl.group) for a in (g32, u32, d32)]
        del g32, u32, d32
        t0 = time.perf_counter()
        wg, wu, wd = (oracle.dequantize(c, sc, b, wl.group) for c, sc, b in logical)
        oracle.mlp_decode(x.values, r.values, wg, wu, wd)
        times.append(time.perf_counter() - t0)
        del wg, wu, wd, logical
    us = float(np.median(times)) * 1e6
    return {
        "value": round(wl.weight_bytes / (us * 1e-6) / 1e9, 3),
        "unit": "GB/s",
        "us_per_layer": round(us, 1),
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"median over {layers} of the 36 layer sets, one 1-row decode each: fp64 dequantize + "
                  f"gate/up + SwiGLU + down + residual (numpy; BLAS threads = cores, elementwise "
                  f"steps single-threaded); host os.cpu_count() = {os.cpu_count()}",
        "us_per_layer_each": [round(t * 1e6, 1) for t in times],
    }


def calibration_copy():
    """A plain 256 MiB device-to-device copy, three times: its FETCH_SIZE / WRITE_SIZE
    readings give the counters' scale."""
    import torch
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# ------------------------------------------------------------------ main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3600)
    ap.add_argument("--warmup", type=int, default=108)
    ap.add_argument("--min-rotations", type=int, default=20,
                    help="whole 36-layer rotations timed at least (the timed steps round up to these)")
    ap.add_argument("--warmup-ms", type=float, default=500.0,
                    help="untimed graph replays before the timed region (milliseconds)")
    ap.add_argument("--event-launches", type=int, default=720)
    ap.add_argument("--cpu-layers", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--samples", type=int, default=20, help="interleaved sampling rounds")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated configuration names, or prefixes ending in '*' "
                         "(e.g. workload5_m*,group_sweep/*): capture and sample only those, skip the "
                         "headline, print their records")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (for scaling HBM counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 "
                                   "(sharding across GPUs is designed, not built)"}))
        return 2

    import torch
    import quantized_decode_mlp_amd as qdm

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    torch.cuda.set_device(0)

    if args.only:
        wanted = [s for s in args.only.split(",") if s]

        def want(name):
            return any(name.startswith(w[:-1]) if w.endswith("*") else name == w for w in wanted)

        builders = (workload_cases, variant_cases, projection_cases)
        cases = [c for b in builders for c in b(want) if want(c.name)]
        if not cases:
            print(json.dumps({"error": f"no configuration matches {args.only!r}"}))
            return 2
        sample_interleaved(cases, args.samples)
        if args.calibration_copy:
            calibration_copy()
        print(json.dumps({"only": args.only, "configs": {c.name: c.record() for c in cases}}), flush=True)
        return 0

    wl = W.WORKLOADS[4]
    n_layers = wl.n_sets
    sets = prepare_sets(wl, n_layers)
    x, r = W.activations(wl, 1)
    xd, rd = _dev(x), _dev(r)
    ws = torch.empty(qdm.mlp_workspace_bytes(1, qdm.QDM_BF16, *sets[0]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(rd)

    def step(i):
        qdm.mlp_decode(xd, rd, *sets[i % n_layers], workspace=ws, out=out)

    # ---- the timed region: W eager steps and, untimed, graph replays for
    # --warmup-ms (the GPU leaves its idle clocks during the host-side
    # preparation only once it is kept busy), then whole rotations of the graph
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_layers):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.warmup_ms * 1e-3:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    rotations = max(args.min_rotations, -(-args.steps // n_layers))
    steps_timed = rotations * n_layers
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(rotations + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for j in range(rotations):
        g.replay()
        ev[j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = ev[0].elapsed_time(ev[-1]) * 1e3 / steps_timed
    rotation_us = [ev[j].elapsed_time(ev[j + 1]) * 1e3 / n_layers for j in range(rotations)]
    us_wall = wall * 1e6 / steps_timed
    gbps = wl.weight_bytes / (us * 1e-6) / 1e9
    _log(f"headline: {us:.3f} us/layer over {steps_timed} steps ({us_wall:.3f} us by the wall clock)")

    # ---- the dominant kernel (gate/up: 2/3 of the bytes), and down, per launch
    h = torch.empty((1, wl.ffn), dtype=torch.float32, device="cuda")
    gu_bytes = 2 * wl.d * wl.ffn * wl.bits // 8 + 8 * (2 * wl.d * wl.ffn // wl.group)
    gu_us = kernel_event_times(lambda i: qdm.gemv_gate_up_swiglu(xd, sets[i][0], h_out=h),
                               n_layers, args.event_launches)
    hd = torch.zeros((1, wl.ffn), dtype=torch.float32, device="cuda")
    dn_us = kernel_event_times(lambda i: qdm.gemv_down_residual(hd, rd, sets[i][1], out=out),
                               n_layers, args.event_launches)
    _log(f"gate/up kernel {gu_us:.2f} us, down kernel {dn_us:.2f} us (graph-replay event means)")
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9

    # cross-check this very launch configuration on a sampled layer
    y_dev = qdm.mlp_decode(xd, rd, *sets[17], workspace=ws, out=torch.empty_like(rd))
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(y_dev.float()).all())

    if args.calibration_copy:
        calibration_copy()

    # ---- every configuration, sampled in interleaved rounds
    cases = headline_cases(sets, wl)
    if not args.no_other_configs:
        cases += workload_cases() + variant_cases() + projection_cases()
    _log(f"{len(cases)} configurations captured; sampling")
    sample_interleaved(cases, args.samples)
    recs = {c.name: c.record() for c in cases}
    interleaved = recs.pop("headline")["us_per_layer"]
    chain = {"workload": "Qwen3-8B-shaped layer as above, with the residual add + RMSNorm (bf16, eps 1e-5) "
                         "that feeds it",
             "add_rmsnorm_then_mlp": recs.pop("decode_chain/add_rmsnorm_then_mlp"),
             "chained": recs.pop("decode_chain/chained")}

    cpu = None
    if not args.no_cpu_baseline:
        _log("timing the fp64 CPU oracle ...")
        cpu = cpu_baseline(wl, args.cpu_layers)
        _log(f"cpu oracle: {cpu['us_per_layer']:.0f} us/layer")

    rec = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "us_per_layer": round(us, 3),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "n_gpus": 1,
        "steps": args.steps,
        "steps_timed": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations x uint8 codes: f16-pair dot products (v_dot2_f32_f16), fp32 accumulation, "
                 "bf16 output",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped MLP decode stack: d=4096, ffn=12288, affine uint8 "
                        "group 128, 36 independent layer sets rotated per call, 1 row, bf16 "
                        "activations and output, fp32 accumulation",
            "d": wl.d, "ffn": wl.ffn, "rows": 1, "bits": wl.bits, "group": wl.group,
            "layer_sets": n_layers, "weight_bytes_per_layer": wl.weight_bytes,
            "launch": f"{rotations} replays of a HIP graph of one 36-layer rotation "
                      f"({steps_timed} steps, HIP events on the launch stream)",
        },
        "wall_us_per_layer": round(us_wall, 3),
        "us_per_layer_samples": pcts(rotation_us),
        "samples": f"per-rotation times of the timed region ({rotations} rotations of {n_layers} layers)",
        "interleaved_us_per_layer": interleaved,
        "kernels_us": {"gemv_gate_up_swiglu": round(gu_us, 3), "gemv_down_residual": round(dn_us, 3)},
        "roofline": {
            "kernel": "gemv_gate_up_swiglu",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": gu_bytes,
        },
        "cpu_baseline": cpu,
        "decode_chain": chain,
        "other_configs": recs,
        "sampling": f"{args.samples} rounds over {len(cases)} configurations, order rotated per round",
        "output_finite": finite,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
