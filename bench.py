#!/usr/bin/env python3
"""Throughput of the weight-only block-32 matmul on one MI355X.

One step = one decode step of the Qwen3-0.6B-shaped decoder at M=1: the 197
GEMVs (28 layers x q, k, v, o, gate, up, down in int4 block-32, plus the tied
lm_head 1024->151936 in int8 block-32) as one grouped launch over a packed,
64-byte-aligned tensor table, issued once per step as a decode loop issues it.
Inputs are resident in HBM before timing starts;
three package copies (1.24 GB) are rotated so every step streams its weights
from HBM rather than from the 256 MB last-level cache.

value = packed weight bytes (codes + binary16 scales) per step / step time
(wall clock over K back-to-back steps, each step one grouped launch issued
directly; the same step replayed from a HIP graph is reported beside it).
The default warmup (500 steps, about 40 ms) brings the chip to its steady
clock state under this load: after idle, the first few hundred back-to-back
launches run up to 20% slower while the clocks settle.
Also reported: the roofline of the grouped GEMV kernel (algorithmic bytes per
launch / the kernel's duration, from HIP events on its stream around the timed
region, one launch per step), the CPU oracle timed on the host cores, and secondary
legs: the sequential and fused (q|k|v, gate|up) forms of the step, tied-
embedding lookups, batched decode of the mixed package at M=1, 2, 4, 8 and 16, the int5
step, and the prefill GEMM (M=4096 gate/up/down int4 + int8 lm_head on the
last 64 rows) in TFLOP/s against the fp16 matrix-core peak. --decode-only
runs the decode-step leg alone (the profile counter runs use it).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 matrix peak, published
COPIES = 3                       # rotated package copies (> 4x the 256 MB cache)
GEMV_SOURCES = ["weight_only_bit_block_amd/csrc/wq_gemv.hip", "weight_only_bit_block_amd/csrc/wq_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_grouped_decode_step_traffic.txt")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary,
    or None when the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha(GEMV_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill GEMM leg")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-step leg (the profile counter runs use this)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a 1 GiB device copy first (counter calibration runs)")
    return ap.parse_args()


def build_decode(torch, wqa, wl, copies):
    """Pack every tensor of the workload into `copies` packages; bind x / y."""
    import numpy as np
    specs = [(t.bits, t.N, t.K) for t in wl.tensors]
    pkgs = [wqa.Package(specs) for _ in range(copies)]
    host_w = {}
    for i, t in enumerate(wl.tensors):
        w = wl.weight(t)
        wd = torch.from_numpy(w).cuda()
        for p in pkgs:
            p.pack_into(i, wd)
        host_w[i] = w if (i < 7 or t.name == "lm_head") else None   # keep a few for the checks
        del wd
    xs_host = {k: wl.activation(k) for k in wl.acts}
    xs_dev = {k: torch.from_numpy(v).cuda() for k, v in xs_host.items()}
    xs = [xs_dev[t.act][t.act_row0: t.act_row0 + t.M] for t in wl.tensors]
    calls, ys = [], []
    for p in pkgs:
        y = [torch.empty((t.M, t.N), dtype=torch.float32, device="cuda") for t in wl.tensors]
        calls.append(wqa.GroupedCall(p, xs, y, wl.M))
        ys.append(y)
    torch.cuda.synchronize()
    return pkgs, calls, ys, host_w, np


def check_outputs(wl, ys, host_w, np, oracle):
    """Outputs of the timed steps: identical across copies, and sampled rows of
    the first seven projections and the lm_head equal to the oracle within the
    GEMV bound."""
    for r in range(1, len(ys)):
        for a, b in zip(ys[0], ys[r]):
            if not bool((a == b).all()):
                raise SystemExit("bench: outputs differ between package copies")
    rng = np.random.Generator(np.random.PCG64(12345))
    worst = 0.0
    for i, w in host_w.items():
        if w is None:
            continue
        t = wl.tensors[i]
        rows = np.sort(rng.choice(t.N, size=min(t.N, 256), replace=False))
        q, s = oracle.quantize(w[rows], t.bits)
        y_ref, B = oracle.matmul(wl.x_for(t), q, s, t.bits)
        y = ys[0][i].cpu().numpy()[:, rows].astype(np.float64)
        err = np.abs(y - y_ref)
        bad = err > 1e-5 * B
        if bad.any():
            raise SystemExit(f"bench: parity failure in {t.name}")
        worst = max(worst, float((err / np.maximum(1e-5 * B, 1e-300)).max()))
    return worst


def cpu_baseline(wl, oracle, np, min_seconds=10.0):
    """The oracle on the host cores over the whole decode step (all 197 GEMVs):
    one warmup pass, then timed passes until at least `min_seconds` of CPU work,
    median reported."""
    packed = []
    wbytes = 0
    for t in wl.tensors:
        q, s = oracle.quantize(wl.weight(t), t.bits)
        packed.append((t, q, s))
        wbytes += q.nbytes + s.nbytes
    times = []
    total = 0.0
    rep = 0
    while rep < 4 or total < min_seconds:
        t0 = time.perf_counter()
        for t, q, s in packed:
            oracle.matmul(wl.x_for(t), q, s, t.bits)
        dt = time.perf_counter() - t0
        if rep > 0:
            times.append(dt)
            total += dt
        rep += 1
    med = sorted(times)[len(times) // 2]
    return {
        "value": round(wbytes / med / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.threads_used(),
        "kind": "oracle",
        "sample": f"the full decode step at M=1 ({len(packed)} GEMVs, {wbytes} packed weight bytes); "
                  f"median of {len(times)} passes after 1 warmup ({total:.1f} s timed), binary64 plain "
                  f"loops, {med:.3f} s per pass",
    }


def sequential_leg(torch, wqa, wl, pkgs, np, steps):
    """The decode step in model order: 197 separate wq_gemv launches, captured
    once in a HIP graph and replayed (launch-bound form of the same work)."""
    xs = {k: torch.from_numpy(wl.activation(k)).cuda() for k in wl.acts}
    xl = [xs[t.act][t.act_row0: t.act_row0 + t.M] for t in wl.tensors]
    graphs, outs = [], []
    for p in pkgs:
        ys = [torch.empty((t.M, t.N), dtype=torch.float32, device="cuda") for t in wl.tensors]

        def run(p=p, ys=ys):
            for i, t in enumerate(wl.tensors):
                wqa.gemv(xl[i], p.q(i), p.scales(i), t.bits, out=ys[i])

        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                run()
        torch.cuda.synchronize()
        graphs.append(g)
        outs.append(ys)
    for i in range(3):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    # every replayed output equals the eager launches of the same package
    for r, p in enumerate(pkgs):
        for i, t in enumerate(wl.tensors):
            ref = wqa.gemv(xl[i], p.q(i), p.scales(i), t.bits)
            if not bool((ref == outs[r][i]).all()):
                raise SystemExit("bench: graph replay differs from eager launches")
    return {"form": "197 wq_gemv launches in model order, one HIP graph per package copy",
            "ms_per_step": round(ms, 5), "weight_gbs": round(wl.weight_bytes / (ms * 1e-3) / 1e9, 1)}


def embed_leg(torch, wqa, wl, pkg, host_w, np, oracle, reps=200):
    """Tied-embedding lookups (wq_embed) from the packed int8 lm_head of the
    decode package: 1 and 128 tokens (the LiteRT card's embed_1 / embed_128) and
    4096 tokens (the long-prefill length). Each size is captured as a graph of
    `reps` lookups and replayed; the looked-up rows are checked bitwise against
    the oracle on the same rows."""
    lm = [i for i, t in enumerate(wl.tensors) if t.name == "lm_head"][0]
    t = wl.tensors[lm]
    q, sc = pkg.q(lm), pkg.scales(lm)
    rng = np.random.Generator(np.random.PCG64(777))
    out = {}
    for n in (1, 128, 4096):
        ids_h = rng.integers(0, t.N, (reps, n)).astype(np.int32)      # a new id set per lookup
        ids = torch.from_numpy(ids_h).cuda()
        y = torch.empty((n, t.K), dtype=torch.float32, device="cuda")
        wqa.embed(ids[0], q, sc, t.K, t.bits, out=y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for r in range(reps):
                    wqa.embed(ids[r], q, sc, t.K, t.bits, out=y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (3 * reps)
        qr, sr = oracle.quantize(host_w[lm][ids_h[-1]], t.bits)      # y holds the last lookup
        ref = oracle.embed(np.arange(n), qr, sr, t.K, t.bits)
        if not np.array_equal(y.cpu().numpy().astype(np.float64), ref):
            raise SystemExit(f"bench: embedding lookup of {n} rows differs from the oracle")
        nbytes = n * (t.K * t.bits // 8 + t.K // 32 * 2 + 4 * t.K + 4)
        out[f"embed_{n}"] = {"us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes": nbytes}
    out["table"] = f"int8 lm_head {t.N}x{t.K}, packed; rows bitwise equal to the oracle"
    return out


def mixed_leg(torch, wqa, inputs, np, oracle, steps, warmup):
    """Batched decode over the mixed package (attention int8, MLP int4, lm_head
    int8), one grouped launch per step at M = 1, 2, 4, 8 and 16 (M <= 2 on the
    fp32-FMA kernel, M >= 3 on the matrix cores)."""
    out = {}
    for M in (1, 2, 4, 8, 16):
        wl = inputs.decode_step(M, mixed=True)
        pkgs, calls, ys, host_w, _ = build_decode(torch, wqa, wl, COPIES)
        launch_ms, wall_ms = time_grouped(torch, calls, steps, warmup)
        worst = check_outputs(wl, ys, host_w, np, oracle)
        del pkgs, calls, ys
        torch.cuda.empty_cache()
        gbs = wl.total_bytes / (launch_ms * 1e-3) / 1e9
        out[f"m{M}"] = {"ms_per_step": round(wall_ms, 5), "launch_ms": round(launch_ms, 5),
                        "weight_gbs": round(wl.weight_bytes / (wall_ms * 1e-3) / 1e9, 1),
                        "algorithmic_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                        "worst_err_over_bound": round(worst, 4)}
    out["workload"] = "decode_step_mixed (attention int8, MLP int4, lm_head int8), 197 GEMVs"
    return out


def int5_leg(torch, wqa, inputs, np, oracle, steps, warmup):
    """INT5 (f4): the decode step with every projection packed in int5 (lm_head
    int8) as one grouped launch, and the M=4096 gate projection in int5 through
    the prefill GEMM."""
    wl = inputs.decode_step(1, proj_bits=5)
    pkgs, calls, ys, host_w, _ = build_decode(torch, wqa, wl, COPIES)
    launch_ms, wall_ms = time_grouped(torch, calls, steps, warmup)
    worst = check_outputs(wl, ys, host_w, np, oracle)
    del pkgs, calls, ys
    torch.cuda.empty_cache()
    out = {"workload": wl.name,
           "decode_grouped": {"ms_per_step": round(wall_ms, 5), "launch_ms": round(launch_ms, 5),
                              "weight_bytes": wl.weight_bytes,
                              "weight_gbs": round(wl.weight_bytes / (wall_ms * 1e-3) / 1e9, 1),
                              "algorithmic_gbs": round(wl.total_bytes / (launch_ms * 1e-3) / 1e9, 1),
                              "hbm_frac": round(wl.total_bytes / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "worst_err_over_bound": round(worst, 4)}}
    lp = inputs.long_prefill()
    t = lp.tensors[0]                                       # gate 1024 -> 3072 at M=4096
    q, sc = wqa.pack(torch.from_numpy(lp.weight(t)).cuda(), 5)
    x = torch.from_numpy(lp.x_for(t)).cuda()
    y = torch.empty((t.M, t.N), dtype=torch.float32, device="cuda")
    for _ in range(3):
        wqa.linear(x, q, sc, 5, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    a.record()
    for _ in range(reps):
        wqa.linear(x, q, sc, 5, out=y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tf = 2 * t.M * t.N * t.K / (ms * 1e-3) / 1e12
    out["gemm_gate_m4096"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                              "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
    return out


def prefill_leg(torch, wqa, inputs, steps, warmup):
    """M=4096 gate/up/down (int4) + int8 lm_head on the last 64 rows, via wq_linear."""
    wl = inputs.long_prefill()
    packed = []
    for t in wl.tensors:
        q, s = wqa.pack(torch.from_numpy(wl.weight(t)).cuda(), t.bits)
        packed.append((q, s))
    xs = {k: torch.from_numpy(wl.activation(k)).cuda() for k in wl.acts}
    outs = [torch.empty((t.M, t.N), dtype=torch.float32, device="cuda") for t in wl.tensors]

    def step():
        for i, t in enumerate(wl.tensors):
            wqa.linear(xs[t.act][t.act_row0: t.act_row0 + t.M], packed[i][0], packed[i][1], t.bits, out=outs[i])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in wl.tensors]
    per = [0.0] * len(wl.tensors)
    t0 = time.perf_counter()
    for _ in range(steps):
        for i, t in enumerate(wl.tensors):
            ev[i][0].record(stream)
            wqa.linear(xs[t.act][t.act_row0: t.act_row0 + t.M], packed[i][0], packed[i][1], t.bits, out=outs[i])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        for i in range(len(wl.tensors)):
            per[i] += ev[i][0].elapsed_time(ev[i][1])
    wall = (time.perf_counter() - t0) / steps
    per = [p / steps for p in per]                         # ms per call
    gemm_idx = [i for i, t in enumerate(wl.tensors) if t.name != "lm_head"]
    mlp_flops = sum(2 * wl.tensors[i].M * wl.tensors[i].N * wl.tensors[i].K for i in gemm_idx)
    mlp_ms = sum(per[i] for i in gemm_idx)
    # the same MLP GEMMs (gate, up, down) in one grouped prefill launch
    mlp = [wl.tensors[i] for i in gemm_idx]
    pkg = wqa.Package([(t.bits, t.N, t.K) for t in mlp])
    for j, t in enumerate(mlp):
        pkg.pack_into(j, torch.from_numpy(wl.weight(t)).cuda())
    gys = [torch.empty((t.M, t.N), dtype=torch.float32, device="cuda") for t in mlp]
    gcall = wqa.GroupedCall(pkg, [xs[t.act][t.act_row0: t.act_row0 + t.M] for t in mlp], gys, mlp[0].M,
                            prefill=True)
    g_ms, _ = time_grouped(torch, [gcall], max(10, 3 * steps), max(3, warmup))
    torch.cuda.synchronize()
    # against the per-call outputs (the down projection's K split differs: fp32
    # summation order only)
    g_diff = max(float(torch.linalg.vector_norm(gys[j] - outs[i]) / torch.linalg.vector_norm(outs[i]))
                 for j, i in enumerate(gemm_idx))
    if not g_diff <= 1e-5:
        log(f"grouped MLP outputs differ from wq_linear's: relative {g_diff:.2e}")
    tflops_grouped = mlp_flops / (g_ms * 1e-3) / 1e12
    lm = [i for i, t in enumerate(wl.tensors) if t.name == "lm_head"][0]
    lt = wl.tensors[lm]
    lm_bytes = lt.weight_bytes + 4 * lt.M * lt.K + 4 * lt.M * lt.N
    # the down projection (K=3072, N=1024) is the dominant-shape check on the MFMA kernel
    tflops_mlp = mlp_flops / (mlp_ms * 1e-3) / 1e12
    return {
        "workload": wl.name,
        "tflops": round(wl.flops / (sum(per) * 1e-3) / 1e12, 2),
        "ms_per_step": round(sum(per), 4),
        "wall_ms_per_step": round(wall * 1e3, 4),
        "mlp_gemm": {"calls": "gate, up, down at M=4096 (int4)", "tflops": round(tflops_mlp, 2),
                     "ms": round(mlp_ms, 4),
                     "roofline": {"bound": "mfma", "achieved": round(tflops_mlp, 2),
                                  "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tflops_mlp / MFMA_F16_PEAK_TFLOPS, 4)}},
        "mlp_gemm_grouped": {"calls": "gate, up, down at M=4096 in one wq_gemm_grouped launch",
                             "tflops": round(tflops_grouped, 2), "ms": round(g_ms, 4),
                             "rel_diff_vs_per_call": g_diff,
                             "frac": round(tflops_grouped / MFMA_F16_PEAK_TFLOPS, 4)},
        "lm_head_m64": {"ms": round(per[lm], 4), "gbs": round(lm_bytes / (per[lm] * 1e-3) / 1e9, 1),
                        "hbm_frac": round(lm_bytes / (per[lm] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def layer_prefill_leg(torch, wqa, inputs, steps, warmup):
    """Prefill through the seven int4 projections of one layer (M = 128 and
    1024): one grouped prefill launch over the layer's tensor table, against the
    seven wq_gemm launches issued back to back."""
    out = {}
    for M in (128, 1024):
        wl = inputs.prefill_layer(M)
        specs = [(t.bits, t.N, t.K) for t in wl.tensors]
        pkg = wqa.Package(specs)
        for i, t in enumerate(wl.tensors):
            pkg.pack_into(i, torch.from_numpy(wl.weight(t)).cuda())
        xs = [torch.from_numpy(wl.x_for(t)).cuda() for t in wl.tensors]
        ys = [torch.empty((M, t.N), dtype=torch.float32, device="cuda") for t in wl.tensors]
        call = wqa.GroupedCall(pkg, xs, ys, M, prefill=True)
        g_ms, _ = time_grouped(torch, [call], steps, warmup)

        def seq():
            for i, t in enumerate(wl.tensors):
                wqa.gemm(xs[i], pkg.q(i), pkg.scales(i), t.bits, out=ys[i])

        s_ms, _ = time_grouped(torch, [seq], steps, warmup)
        flops = sum(2 * M * t.N * t.K for t in wl.tensors)
        out[f"m{M}"] = {"grouped_ms": round(g_ms, 5), "grouped_tflops": round(flops / (g_ms * 1e-3) / 1e12, 2),
                        "sequential_ms": round(s_ms, 5),
                        "sequential_tflops": round(flops / (s_ms * 1e-3) / 1e12, 2),
                        "workgroups": call.total_tiles}
    out["note"] = ("7 int4 projections (q, k, v, o, gate, up, down) of one layer, 1% outlier rows; "
                   "grouped = wq_gemm_grouped, one launch; sequential = 7 wq_gemm launches; HIP events")
    return out


def time_grouped(torch, calls, steps, warmup):
    """A step is one grouped launch (the whole decode step), issued directly on
    the current stream as a decode loop issues it; the timed region runs `steps`
    steps back to back, rotating the package copies. Returns (ms per step from
    HIP events on that stream, wall-clock ms per step)."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        calls[i % len(calls)]()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall * 1e3 / steps


def graph_step_ms(torch, calls, steps):
    """The same step captured once per package copy in a HIP graph and replayed
    once per step (graph-launch gaps included), HIP events per step."""
    graphs = []
    for c in calls:
        c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                c()
        torch.cuda.synchronize()
        graphs.append(g)
    stream = torch.cuda.current_stream()
    for i in range(3):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def fused_leg(torch, wqa, inputs, np, oracle, steps, warmup):
    """Shared-input fusion: the same decode step with q|k|v and gate|up stacked
    along N (113 GEMVs): one grouped launch, and 113 launches in model order."""
    wl = inputs.decode_step(1, fused=True)
    pkgs, calls, ys, host_w, _ = build_decode(torch, wqa, wl, COPIES)
    launch_ms, wall_ms = time_grouped(torch, calls, steps, warmup)
    worst = check_outputs(wl, ys, host_w, np, oracle)
    seq = sequential_leg(torch, wqa, wl, pkgs, np, max(10, steps // 4))
    seq["form"] = f"{len(wl.tensors)} wq_gemv launches in model order, one HIP graph per package copy"
    out = {"workload": wl.name, "gemvs": len(wl.tensors),
           "grouped": {"ms_per_step": round(wall_ms, 5), "launch_ms": round(launch_ms, 5),
                       "weight_gbs": round(wl.weight_bytes / (wall_ms * 1e-3) / 1e9, 1)},
           "sequential": seq, "worst_err_over_bound": round(worst, 4)}
    del pkgs, calls, ys
    torch.cuda.empty_cache()
    return out


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the path runs on one GPU and multi-GPU runs are not part of this build.", file=sys.stderr)
        return 2

    import torch
    import weight_only_bit_block_amd as wqa
    from weight_only_bit_block_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wqa.load()

    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = inputs.decode_step(1)
    log(f"packing {len(wl.tensors)} tensors x {COPIES} copies ({wl.weight_bytes} B each)")
    pkgs, calls, ys, host_w, np = build_decode(torch, wqa, wl, COPIES)

    log(f"timing {args.steps} decode steps")
    step_ms, ms_per_step = time_grouped(torch, calls, args.steps, args.warmup)
    launch_ms = step_ms
    graph_ms = graph_step_ms(torch, calls, args.steps)
    value = wl.weight_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = wl.total_bytes / (launch_ms * 1e-3) / 1e9
    traffic = read_traffic()

    import oracle
    worst = check_outputs(wl, ys, host_w, np, oracle)
    log(f"timed outputs checked (worst err/bound {worst:.3f})")
    seq = emb = None
    if not args.decode_only:
        log("sequential form (hipGraph of 197 launches)")
        seq = sequential_leg(torch, wqa, wl, pkgs, np, max(10, args.steps // 4))
        log("tied-embedding lookups")
        emb = embed_leg(torch, wqa, wl, pkgs[0], host_w, np, oracle)
    del pkgs, calls, ys
    torch.cuda.empty_cache()

    result = {
        "metric": "W-only int4/int8 GEMV weight GB/s (M=1) + prefill GEMM TFLOPS, % roofline",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name,
                   "description": "one decode step at M=1: 196 int4 block-32 GEMVs (28 layers x q 1024->2048, "
                                  "k/v 1024->1024, o 2048->1024, gate/up 1024->3072, down 3072->1024) + "
                                  "int8 block-32 lm_head 1024->151936, one grouped launch",
                   "weight_bytes_per_step": wl.weight_bytes,
                   "algorithmic_bytes_per_step": wl.total_bytes,
                   "package_copies_rotated": COPIES},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic) if traffic is not None else None),
                     "kernel": "gemv_grouped_kernel", "launch_ms": round(launch_ms, 5),
                     "launch_ms_source": "HIP events on the launch stream around the timed region "
                                         "(one grouped launch per step), divided by the steps",
                     "step_graph_replay_ms": round(graph_ms, 5),
                     "bytes_per_launch": wl.total_bytes},
        "parity": {"timed_outputs": "copies bitwise equal; sampled rows within 1e-5*sum|x||w|",
                   "worst_err_over_bound": round(worst, 4)},
        "decode_step_sequential": seq,
        "embedding": emb,
    }
    if not args.decode_only:
        log("shared-input fusion (113 GEMVs)")
        result["decode_step_fused"] = fused_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup)
        log("mixed package, batched decode (M = 1, 2, 4, 8, 16)")
        result["decode_step_mixed"] = mixed_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup)
        log("int5 decode step and GEMM")
        result["int5"] = int5_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup)
    if not args.no_prefill and not args.decode_only:
        log("prefill leg")
        result["prefill"] = prefill_leg(torch, wqa, inputs, max(3, args.steps // 10), max(1, args.warmup // 10))
        log("layer prefill leg (grouped prefill launch)")
        result["layer_prefill"] = layer_prefill_leg(torch, wqa, inputs, max(20, args.steps // 5),
                                                    max(5, args.warmup // 5))
    if not args.no_cpu_baseline and not args.decode_only:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, oracle, np)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
