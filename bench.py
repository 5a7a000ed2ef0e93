"""Benchmark of the one-row quantized decode MLP on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the Qwen3-8B-shaped MLP stack -- d = 4096, ffn = 12288, affine
uint8 weights with groups of 128 along the input dim, 36 independent layer
weight sets (5.78 GB, far beyond the 256 MB Infinity Cache and the L2s)
resident in HBM and rotated per call, 1 activation row in bf16.
One step = one MLP layer decode: the gate/up + SwiGLU kernel and the
down + residual kernel on layer (step mod 36).  Steps are replayed from a
HIP graph holding one rotation of 36 layers (the launch-bound inner loop);
an eager Python-launched pass is timed too and reported beside it.  The
dominant kernel's duration comes from HIP events around graph replays of
that kernel alone.

Prints one JSON line: metric, value (weight-stream GB/s = algorithmic weight
bytes per layer / time per layer), the time per layer (and its p10/p50/p90
over single-rotation samples), the fraction of the 8 TB/s HBM peak, a
roofline record for the dominant kernel (gate/up), the fp64 CPU oracle timed
on a bounded sample on the host cores, and (unless --no-other-configs) the
other workloads: Llama-3.2-1B uint8, Qwen2.5-1.5B bf16, Llama-3-8B 4-bit at
1, 4 and 16 rows (with matrix-core utilisation), add+RMSNorm and a launch
floor.
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


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prepare_sets(wl: W.Workload, n_sets: int):
    """Draws, quantizes and packs n_sets weight sets on host threads and uploads them."""
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
            gu = qdm.Weight.from_host(wl.ffn, wl.d, wl.bits, wl.group, q, sb)
            dn = qdm.Weight.from_host(wl.d, wl.ffn, wl.bits, wl.group, dq, dsb)
            sets[s] = (gu, dn)
            if (s + 1) % 6 == 0 or s + 1 == n_sets:
                _log(f"prepared {s + 1}/{n_sets} layer sets ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    return sets


def time_steps(run_step, n_layers, steps, warmup, use_graph):
    """Times exactly `steps` layer steps; returns seconds."""
    import torch
    for i in range(warmup):
        run_step(i % n_layers)
    torch.cuda.synchronize()
    if not use_graph:
        t0 = time.perf_counter()
        for i in range(steps):
            run_step(i % n_layers)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_layers):
            run_step(i)
    g.replay()
    torch.cuda.synchronize()
    full, rest = divmod(steps, n_layers)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(full):
        g.replay()
    for i in range(rest):
        run_step(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, g


def kernel_event_times(launch, n_layers, launches):
    """Average device duration of one kernel: a HIP graph of n_layers back-to-back
    launches (rotating over the layer sets) is replayed between two HIP events
    recorded on the stream the kernels run on (torch's current stream); the
    elapsed time over the launches.  Graph launches on one stream leave gaps of
    well under 1 % of these kernels' durations, so this tracks the profiler's
    per-dispatch average."""
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


def graph_samples(run_step, n_layers, samples):
    """Per-layer times (us) of `samples` replays of one graph rotation over the
    n_layers layer sets, each bracketed by HIP events on the launch stream."""
    import torch
    for i in range(n_layers):
        run_step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_layers):
            run_step(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        out.append(a.elapsed_time(b) / n_layers * 1e3)
    return out


def pcts(v):
    return {"p10": round(float(np.percentile(v, 10)), 3), "p50": round(float(np.percentile(v, 50)), 3),
            "p90": round(float(np.percentile(v, 90)), 3)}


def other_configs(samples, only=None):
    """The other workloads' decode MLP (and the add+RMSNorm row), each over address-distinct
    weight copies of at least 2 GiB so no weight byte is served from a cache.  `only`
    (workload index, rows) restricts it to that one MLP, e.g. for a kernel profile."""
    import torch
    import quantized_decode_mlp_amd as qdm
    res = {}
    torch_dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

    def dev(a):
        t = torch.from_numpy(a.raw) if a.dtype == "f32" else \
            torch.from_numpy(a.raw.view(np.int16)).view(torch_dt[a.dtype])
        return t.cuda()

    for wi in ((only[0],) if only else (2, 3, 5)):
        wl = W.WORKLOADS[wi]
        g32, u32, d32 = W.weights_f32(wl, 0)
        if wl.bits == 16:
            gb, ub, db = (W.to_storage(a, "bf16").raw for a in (g32, u32, d32))
            q, sb, dq, dsb = qdm.pack_dense_gate_up(gb, ub), None, db, None
        else:
            q, sb = qdm.quantize_pack_gate_up(g32, u32, wl.bits, wl.group)
            dq, dsb = qdm.quantize_pack_rows(d32, wl.bits, wl.group)
        del g32, u32, d32
        copies = int(-(-(2 << 30) // wl.weight_bytes))
        sets = [(qdm.Weight.from_host(wl.ffn, wl.d, wl.bits, wl.group, q, sb),
                 qdm.Weight.from_host(wl.d, wl.ffn, wl.bits, wl.group, dq, dsb)) for _ in range(copies)]
        for m in ((only[1],) if only else (wl.rows + (128, 512) if wi == 5 else (1,))):
            x, r = W.activations(wl, m)
            xd, rd = dev(x), dev(r)
            ws = torch.empty(qdm.mlp_workspace_bytes(m, wl.ffn), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(rd)
            t = graph_samples(lambda i: qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out), copies, samples)
            med = float(np.median(t))
            rec = {"us_per_layer": pcts(t), "weight_GBps": round(wl.weight_bytes / (med * 1e-6) / 1e9, 1),
                   "hbm_frac": round(wl.weight_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4), "copies": copies}
            if m > 1:
                flops = 2 * m * 3 * wl.d * wl.ffn
                rec["mfma_util_bf16"] = round(flops / (med * 1e-6) / 2.5e15, 5)
                rec["tflops"] = round(flops / (med * 1e-6) / 1e12, 2)
            res[f"workload{wi}_m{m}"] = rec
            _log(f"workload {wi} m={m}: {med:.2f} us/layer")
        del sets
        torch.cuda.empty_cache()
    if only:
        return res
    res.update(projection_configs(samples, dev))
    res["group_sweep"] = group_sweep(samples, dev)
    res["bf16_scale_bias"] = sb16_configs(samples, dev)
    res.update(mx_configs(samples, dev))
    # add + RMSNorm (the row-a5 kernel) on the Llama-3.2-1B-shaped f16 row, and a launch floor
    wl = W.WORKLOADS[2]
    a, b, w = W.rmsnorm_inputs(wl)
    ad, bd, wd = dev(a), dev(b), dev(w)
    so, no = torch.empty_like(ad), torch.empty_like(ad)
    t = graph_samples(lambda i: qdm.add_rmsnorm(ad, bd, wd, wl.norm_eps, s_out=so, n_out=no), 36, samples)
    res["add_rmsnorm_f16_2048"] = {"us": pcts(t)}
    z = torch.empty(1, device="cuda")
    t = graph_samples(lambda i: z.zero_(), 36, samples)
    res["launch_floor_fill_kernel"] = {"us": pcts(t)}
    return res


def group_sweep(samples, dev):
    """The one-row MLP of each quantized workload shape at affine groups 32, 64 and 128 (the
    groups the pages race per shape), over address-distinct copies of at least 2 GiB."""
    import torch
    import quantized_decode_mlp_amd as qdm
    res = {}
    for wi in (2, 4, 5):
        wl = W.WORKLOADS[wi]
        g32, u32, d32 = W.weights_f32(wl, 0)
        x, r = W.activations(wl, 1)
        xd, rd = dev(x), dev(r)
        ws = torch.empty(qdm.mlp_workspace_bytes(1, wl.ffn), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(rd)
        row = {}
        for group in (32, 64, 128):
            q, sb = qdm.quantize_pack_gate_up(g32, u32, wl.bits, group)
            dq, dsb = qdm.quantize_pack_rows(d32, wl.bits, group)
            n_w = 3 * wl.d * wl.ffn
            nbytes = n_w * wl.bits // 8 + 8 * (n_w // group)
            copies = int(-(-(2 << 30) // nbytes))
            sets = [(qdm.Weight.from_host(wl.ffn, wl.d, wl.bits, group, q, sb),
                     qdm.Weight.from_host(wl.d, wl.ffn, wl.bits, group, dq, dsb)) for _ in range(copies)]
            del q, sb, dq, dsb
            t = graph_samples(lambda i: qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out), copies, samples)
            med = float(np.median(t))
            row[f"g{group}"] = {"us_per_layer": round(med, 3), "weight_bytes": nbytes,
                                "weight_GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
            _log(f"group sweep workload {wi} g{group}: {med:.2f} us/layer")
            del sets
            torch.cuda.empty_cache()
        res[f"workload{wi}_m1"] = row
        del g32, u32, d32
    return res


def mx_configs(samples, dev):
    """The Qwen3-8B-shaped one-row MLP with MXFP8 and MXFP4 block-scaled weights, and the
    Llama-3-8B-shaped MLP in MXFP4 at 1, 4 and 16 rows, over address-distinct copies of at
    least 2 GiB."""
    import torch
    import quantized_decode_mlp_amd as qdm
    res = {}
    wl = W.WORKLOADS[4]
    g32, u32, d32 = W.weights_f32(wl, 0)
    x, r = W.activations(wl, 1)
    xd, rd = dev(x), dev(r)
    ws = torch.empty(qdm.mlp_workspace_bytes(1, wl.ffn), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(rd)
    for name, fmt in (("mxfp8", qdm.QDM_MXFP8), ("mxfp4", qdm.QDM_MXFP4)):
        q, e = qdm.quantize_mx_gate_up(g32, u32, fmt)
        dq, de = qdm.quantize_mx(d32, fmt)
        nbytes = 2 * q.nbytes // 2 + e.nbytes + dq.nbytes + de.nbytes
        copies = int(-(-(2 << 30) // nbytes))
        sets = [(qdm.Weight.from_host(wl.ffn, wl.d, fmt, 32, q, None, block_scales=e),
                 qdm.Weight.from_host(wl.d, wl.ffn, fmt, 32, dq, None, block_scales=de)) for _ in range(copies)]
        t = graph_samples(lambda i: qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out), copies, samples)
        med = float(np.median(t))
        res[f"qwen3_8b_{name}_m1"] = {"us_per_layer": pcts(t), "weight_bytes": int(nbytes),
                                      "weight_GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                      "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                      "copies": copies}
        _log(f"{name}: {med:.2f} us/layer")
        del sets
        torch.cuda.empty_cache()
    del g32, u32, d32
    # the Llama-3-8B-shaped layer in MXFP4 at 1, 4 and 16 rows
    wl = W.WORKLOADS[5]
    g32, u32, d32 = W.weights_f32(wl, 0)
    fmt = qdm.QDM_MXFP4
    q, e = qdm.quantize_mx_gate_up(g32, u32, fmt)
    dq, de = qdm.quantize_mx(d32, fmt)
    del g32, u32, d32
    nbytes = q.nbytes + e.nbytes + dq.nbytes + de.nbytes
    copies = int(-(-(2 << 30) // nbytes))
    sets = [(qdm.Weight.from_host(wl.ffn, wl.d, fmt, 32, q, None, block_scales=e),
             qdm.Weight.from_host(wl.d, wl.ffn, fmt, 32, dq, None, block_scales=de)) for _ in range(copies)]
    for m in wl.rows:
        x, r = W.activations(wl, m)
        xd, rd = dev(x), dev(r)
        ws = torch.empty(qdm.mlp_workspace_bytes(m, wl.ffn), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(rd)
        try:
            t = graph_samples(lambda i: qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out), copies, samples)
        except qdm.QdmError as err:
            res[f"llama3_8b_mxfp4_m{m}"] = {"unsupported": str(err)}
            continue
        med = float(np.median(t))
        res[f"llama3_8b_mxfp4_m{m}"] = {"us_per_layer": pcts(t), "weight_bytes": int(nbytes),
                                        "weight_GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                        "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                        "copies": copies}
        _log(f"llama3_8b mxfp4 m={m}: {med:.2f} us/layer")
    del sets
    torch.cuda.empty_cache()
    return res


def sb16_configs(samples, dev):
    """Each quantized workload's MLP with its (scale, bias) pairs stored as bf16 (the
    QDM_U8_SB16 / QDM_U4_SB16 formats), over address-distinct copies of at least 2 GiB."""
    import torch
    import quantized_decode_mlp_amd as qdm
    res = {}
    for wi in (2, 4, 5):
        wl = W.WORKLOADS[wi]
        g32, u32, d32 = W.weights_f32(wl, 0)
        q, sb = qdm.quantize_pack_gate_up_sb16(g32, u32, wl.bits, wl.group)
        dq, dsb = qdm.quantize_pack_rows_sb16(d32, wl.bits, wl.group)
        del g32, u32, d32
        fmt = qdm.QDM_U8_SB16 if wl.bits == 8 else qdm.QDM_U4_SB16
        nbytes = q.nbytes + sb.nbytes + dq.nbytes + dsb.nbytes
        copies = int(-(-(2 << 30) // nbytes))
        sets = [(qdm.Weight.from_host(wl.ffn, wl.d, fmt, wl.group, q, sb),
                 qdm.Weight.from_host(wl.d, wl.ffn, fmt, wl.group, dq, dsb)) for _ in range(copies)]
        for m in ((1, 4, 16) if wi == 5 else (1,)):
            x, r = W.activations(wl, m)
            xd, rd = dev(x), dev(r)
            ws = torch.empty(qdm.mlp_workspace_bytes(m, wl.ffn), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(rd)
            t = graph_samples(lambda i: qdm.mlp_decode(xd, rd, *sets[i], workspace=ws, out=out), copies, samples)
            med = float(np.median(t))
            res[f"workload{wi}_m{m}"] = {"us_per_layer": pcts(t), "weight_bytes": int(nbytes),
                                         "weight_GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                         "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                                         "copies": copies}
            _log(f"bf16 pairs workload {wi} m={m}: {med:.2f} us/layer")
        del sets
        torch.cuda.empty_cache()
    return res


def projection_configs(samples, dev):
    """One-row projections other than the MLP: the Qwen3-8B-shaped lm_head (vocab 151936), and
    the four attention projections of a Qwen2.5-1.5B-shaped layer (q/k/v with bias, o without),
    each over address-distinct weight copies of at least 2 GiB."""
    import torch
    import quantized_decode_mlp_amd as qdm
    res = {}

    def prepared(p):
        w32, b, x = W.projection_inputs(p, 1)
        q, sb = qdm.quantize_pack_rows(w32, p.bits, p.group)
        return q, sb, (None if b is None else dev(b)), dev(x)

    p = W.PROJECTIONS["qwen3_8b_lm_head"]
    q, sb, _, xd = prepared(p)
    copies = int(-(-(2 << 30) // p.weight_bytes))
    ws = [qdm.Weight.from_host(p.n, p.k, p.bits, p.group, q, sb) for _ in range(copies)]
    del q, sb
    out = torch.empty((1, p.n), dtype=xd.dtype, device="cuda")
    t = graph_samples(lambda i: qdm.gemv_linear(xd, ws[i], out=out), copies, samples)
    med = float(np.median(t))
    res["lm_head_qwen3_8b"] = {"us": pcts(t), "weight_GBps": round(p.weight_bytes / (med * 1e-6) / 1e9, 1),
                               "hbm_frac": round(p.weight_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                               "copies": copies}
    _log(f"lm_head: {med:.2f} us")
    del ws
    torch.cuda.empty_cache()

    keys = ("qwen25_1p5b_q", "qwen25_1p5b_k", "qwen25_1p5b_v", "qwen25_1p5b_o")
    prep = [prepared(W.PROJECTIONS[k]) for k in keys]
    layer_bytes = sum(W.PROJECTIONS[k].weight_bytes for k in keys)
    copies = int(-(-(2 << 30) // layer_bytes))
    layers = [[(qdm.Weight.from_host(W.PROJECTIONS[k].n, W.PROJECTIONS[k].k, W.PROJECTIONS[k].bits,
                                     W.PROJECTIONS[k].group, q, sb), bd)
               for k, (q, sb, bd, _) in zip(keys, prep)] for _ in range(copies)]
    xd = prep[0][3]
    outs = [torch.empty((1, W.PROJECTIONS[k].n), dtype=xd.dtype, device="cuda") for k in keys]

    def attn(i):
        for (wt, bd), o in zip(layers[i], outs):
            qdm.gemv_linear(xd, wt, bias=bd, out=o)

    t = graph_samples(attn, copies, samples)
    med = float(np.median(t))
    res["attention_qkvo_qwen25_1p5b"] = {"us_per_layer": pcts(t), "launches": 4,
                                         "weight_GBps": round(layer_bytes / (med * 1e-6) / 1e9, 1),
                                         "copies": copies}
    _log(f"attention q/k/v/o: {med:.2f} us per layer")
    del layers
    torch.cuda.empty_cache()

    # the same projections with q, k and v as one weight (packed rows and their
    # pairs concatenated: every row is quantized on its own) and o: 2 launches
    n_qkv = sum(W.PROJECTIONS[k].n for k in keys[:3])
    qkv_q = np.ascontiguousarray(np.concatenate([prep[j][0] for j in range(3)], axis=0))
    qkv_sb = np.ascontiguousarray(np.concatenate([prep[j][1] for j in range(3)], axis=0))
    qkv_b = torch.cat([prep[j][2] for j in range(3)])
    po = W.PROJECTIONS[keys[3]]
    fused = [(qdm.Weight.from_host(n_qkv, po.k, po.bits, po.group, qkv_q, qkv_sb),
              qdm.Weight.from_host(po.n, po.k, po.bits, po.group, prep[3][0], prep[3][1])) for _ in range(copies)]
    o_qkv = torch.empty((1, n_qkv), dtype=xd.dtype, device="cuda")

    def attn_fused(i):
        qdm.gemv_linear(xd, fused[i][0], bias=qkv_b, out=o_qkv)
        qdm.gemv_linear(xd, fused[i][1], bias=prep[3][2], out=outs[3])

    t = graph_samples(attn_fused, copies, samples)
    med = float(np.median(t))
    res["attention_fused_qkv_o_qwen25_1p5b"] = {"us_per_layer": pcts(t), "launches": 2,
                                                "weight_GBps": round(layer_bytes / (med * 1e-6) / 1e9, 1),
                                                "copies": copies}
    _log(f"attention fused qkv + o: {med:.2f} us per layer")
    del fused
    torch.cuda.empty_cache()
    return res


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
    """The fp64 oracle (as it stands) on `layers` of the workload's layer sets:
    dequantize the layer's codes, both projections, SwiGLU, residual.  The
    oracle's own quantization of those layers is setup, not timed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    x, r = W.activations(wl, 1)
    total = 0.0
    for s in range(layers):
        g32, u32, d32 = W.weights_f32(wl, s)
        logical = [oracle.quantize_affine(a, wl.bits, wl.group) for a in (g32, u32, d32)]
        del g32, u32, d32
        t0 = time.perf_counter()
        wg, wu, wd = (oracle.dequantize(c, sc, b, wl.group) for c, sc, b in logical)
        oracle.mlp_decode(x.values, r.values, wg, wu, wd)
        total += time.perf_counter() - t0
        del wg, wu, wd, logical
    us = total / layers * 1e6
    return {
        "value": round(wl.weight_bytes / (us * 1e-6) / 1e9, 3),
        "unit": "GB/s",
        "us_per_layer": round(us, 1),
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{layers} of the 36 layer sets, one 1-row decode each: fp64 dequantize + "
                  f"gate/up + SwiGLU + down + residual (numpy; BLAS threads = cores, elementwise "
                  f"steps single-threaded); host os.cpu_count() = {os.cpu_count()}",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3600)
    ap.add_argument("--warmup", type=int, default=108)
    ap.add_argument("--event-launches", type=int, default=720)
    ap.add_argument("--cpu-layers", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--samples", type=int, default=20, help="graph-rotation samples for percentiles")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--rows-only", type=int, default=0, metavar="M",
                    help="only the Llama-3-8B-shaped MLP at M rows (graph replays), then exit")
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
    if args.rows_only:
        rec = other_configs(args.samples, only=(5, args.rows_only))
        print(json.dumps({"workload": W.WORKLOADS[5].name, "rows": args.rows_only, **rec}))
        return 0
    wl = W.WORKLOADS[4]
    n_layers = wl.n_sets
    sets = prepare_sets(wl, n_layers)

    x, r = W.activations(wl, 1)
    xd = torch.from_numpy(x.raw.view(np.int16)).view(torch.bfloat16).cuda()
    rd = torch.from_numpy(r.raw.view(np.int16)).view(torch.bfloat16).cuda()
    ws = torch.empty(qdm.mlp_workspace_bytes(1, wl.ffn), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(rd)
    h = torch.empty((1, wl.ffn), dtype=torch.float32, device="cuda")

    def step(i):
        gu, dn = sets[i]
        qdm.mlp_decode(xd, rd, gu, dn, workspace=ws, out=out)

    # eager (Python-launched) pass
    t_eager, _ = time_steps(step, n_layers, args.steps, args.warmup, use_graph=False)
    us_eager = t_eager / args.steps * 1e6
    _log(f"eager: {us_eager:.2f} us/layer")
    t, us_graph = t_eager, None
    if not args.no_graph:
        t_graph, _ = time_steps(step, n_layers, args.steps, args.warmup, use_graph=True)
        us_graph = t_graph / args.steps * 1e6
        _log(f"graph: {us_graph:.2f} us/layer")
        t = t_graph
    us = t / args.steps * 1e6
    gbps = wl.weight_bytes / (us * 1e-6) / 1e9
    spread = pcts(graph_samples(step, n_layers, args.samples))

    # dominant kernel (gate/up: 2/3 of the bytes), per-launch events
    gu_bytes = 2 * wl.d * wl.ffn * wl.bits // 8 + 8 * (2 * wl.d * wl.ffn // wl.group)
    dn_bytes = wl.weight_bytes - gu_bytes
    gu_us = kernel_event_times(lambda i: qdm.gemv_gate_up_swiglu(xd, sets[i][0], h_out=h),
                               n_layers, args.event_launches)
    hd = torch.zeros((1, wl.ffn), dtype=torch.float32, device="cuda")
    dn_us = kernel_event_times(lambda i: qdm.gemv_down_residual(hd, rd, sets[i][1], out=out),
                               n_layers, args.event_launches)
    _log(f"gate/up kernel {gu_us:.2f} us, down kernel {dn_us:.2f} us (graph-replay event means)")
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9

    # cross-check parity of this very launch configuration on a sampled layer
    y_dev = qdm.mlp_decode(xd, rd, *sets[17], workspace=ws, out=torch.empty_like(rd))
    torch.cuda.synchronize()
    y_sample = y_dev.float().cpu().numpy()
    finite = bool(np.all(np.isfinite(y_sample)))

    if args.calibration_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE give the counters' scale
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the decode chain on the same 36 layer sets: add + RMSNorm then the MLP
    # (three launches) against the chained call (two launches)
    a, b, nw = W.chain_inputs(wl, 1)
    ad, bd, nwd = (torch.from_numpy(v.raw.view(np.int16)).view(torch.bfloat16).cuda() for v in (a, b, nw))
    so, no = torch.empty_like(ad), torch.empty_like(ad)
    ws_c = torch.empty(qdm.mlp_rmsnorm_workspace_bytes(1, wl.d, wl.ffn, qdm.QDM_BF16), dtype=torch.uint8,
                       device="cuda")

    def sep(i):
        qdm.add_rmsnorm(ad, bd, nwd, wl.norm_eps, s_out=so, n_out=no)
        qdm.mlp_decode(no, so, *sets[i], workspace=ws, out=out)

    t_sep = graph_samples(sep, n_layers, args.samples)
    t_chain = graph_samples(lambda i: qdm.mlp_decode_rmsnorm(ad, bd, nwd, wl.norm_eps, *sets[i], workspace=ws_c,
                                                             s_out=so, out=out), n_layers, args.samples)
    chain = {"workload": "Qwen3-8B-shaped layer as above, with the residual add + RMSNorm (bf16, eps 1e-5) "
                         "that feeds it",
             "add_rmsnorm_then_mlp_us_per_layer": pcts(t_sep), "chained_us_per_layer": pcts(t_chain)}
    _log(f"decode chain: {np.median(t_sep):.2f} us separate, {np.median(t_chain):.2f} us chained")

    others = None
    if not args.no_other_configs:
        others = other_configs(args.samples)

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
        "warmup": args.warmup,
        "ms_per_step": round(t / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped MLP decode stack: d=4096, ffn=12288, affine uint8 "
                        "group 128, 36 independent layer sets rotated per call, 1 row, bf16 "
                        "activations and output, fp32 accumulation",
            "d": wl.d, "ffn": wl.ffn, "rows": 1, "bits": wl.bits, "group": wl.group,
            "layer_sets": n_layers, "weight_bytes_per_layer": wl.weight_bytes,
            "launch": "hip graph of 36 layers" if us_graph is not None else "eager",
        },
        "us_per_layer_samples": spread,
        "eager_us_per_layer": round(us_eager, 3),
        "graph_us_per_layer": None if us_graph is None else round(us_graph, 3),
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
        "other_configs": others,
        "output_finite": finite,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
