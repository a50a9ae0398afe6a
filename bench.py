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
region, one launch per step), the CPU oracle timed on the host cores (all of
them and one), and secondary legs: the single GEMV over 512 distinct weight
copies with the launch floor beside it, the sequential and fused (q|k|v,
gate|up) forms of the step, tied-embedding lookups, batched decode of the mixed
package at M=1, 2, 4, 8 and 16, the int5 step, and the prefill GEMMs (M=4096
gate/up/down int4 + int8 lm_head on the last 64 rows; one layer's seven
projections at M=128 and 1024) in TFLOP/s against the fp16 matrix-core peak.
Prefill numbers are cold: a 1 GiB read-only flush runs before every timed
call (median of --prefill-reps); warm numbers are labelled as such. Every
timed output is NaN-filled first and checked against the oracle on sampled
rows and columns afterwards. --decode-only runs the decode-step leg alone and
--prefill-only the prefill legs alone (the profile counter runs use them).

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
GEMV_SOURCES = ["weight_only_bit_block_amd/csrc/wq_gemv.hip", "weight_only_bit_block_amd/csrc/wq_internal.h",
                "weight_only_bit_block_amd/csrc/wq_device.h",
                "weight_only_bit_block_amd/csrc/wq_decode.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_grouped_decode_step_traffic.txt")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(paths) -> str:
    """Hash of the kernel sources and the compiler flags they are built with."""
    from weight_only_bit_block_amd import build as wq_build
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    h.update(" ".join(wq_build.FLAGS[:-2]).encode())      # the flags, without the include path
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
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill legs, printed as one JSON object (the GEMM counter runs use this)")
    ap.add_argument("--prefill-reps", type=int, default=21,
                    help="cold runs per prefill measurement (median reported)")
    ap.add_argument("--mixed-only", type=int, default=0, metavar="M",
                    help="only the mixed decode leg at this M, printed as one JSON object "
                         "(the matrix-core GEMV counter runs use this)")
    return ap.parse_args()


SAMPLE_ROWS = 16      # weight rows of every tensor checked against the oracle after timing


def build_decode(torch, wqa, wl, copies):
    """Pack every tensor of the workload into `copies` packages; bind x / y (y
    starts as NaN, so an output a kernel skipped cannot pass the checks). Keeps
    SAMPLE_ROWS random weight rows of every tensor for the oracle check."""
    import numpy as np
    specs = [(t.bits, t.N, t.K) for t in wl.tensors]
    pkgs = [wqa.Package(specs) for _ in range(copies)]
    rng = np.random.Generator(np.random.PCG64(12345))
    host_w = {}
    for i, t in enumerate(wl.tensors):
        w = wl.weight(t)
        wd = torch.from_numpy(w).cuda()
        for p in pkgs:
            p.pack_into(i, wd)
        rows = np.sort(rng.choice(t.N, size=min(t.N, SAMPLE_ROWS if t.name != "lm_head" else 256), replace=False))
        host_w[i] = (rows, w[rows].copy())
        del wd, w
    xs_host = {k: wl.activation(k) for k in wl.acts}
    xs_dev = {k: torch.from_numpy(v).cuda() for k, v in xs_host.items()}
    xs = [xs_dev[t.act][t.act_row0: t.act_row0 + t.M] for t in wl.tensors]
    calls, ys = [], []
    for p in pkgs:
        y = [torch.full((t.M, t.N), float("nan"), dtype=torch.float32, device="cuda") for t in wl.tensors]
        calls.append(wqa.GroupedCall(p, xs, y, wl.M))
        ys.append(y)
    torch.cuda.synchronize()
    return pkgs, calls, ys, host_w, np


def check_outputs(wl, ys, host_w, np, oracle):
    """Outputs of the timed steps: identical across copies (every copy ran),
    and sampled rows of every one of the tensors within the GEMV bound of the
    oracle (so no tensor of the timed step was skipped)."""
    for r in range(1, len(ys)):
        for a, b in zip(ys[0], ys[r]):
            if not bool((a == b).all()):
                raise SystemExit("bench: outputs differ between package copies")
    worst = 0.0
    for i, (rows, w) in host_w.items():
        t = wl.tensors[i]
        q, s = oracle.quantize(w, t.bits)
        y_ref, B = oracle.matmul(wl.x_for(t), q, s, t.bits)
        y = ys[0][i][:, rows].cpu().numpy().astype(np.float64)
        err = np.abs(y - y_ref)
        if not np.all(np.isfinite(y)) or bool((err > 1e-5 * B).any()):
            raise SystemExit(f"bench: parity failure in {t.name}")
        worst = max(worst, float((err / np.maximum(1e-5 * B, 1e-300)).max()))
    return worst


def cpu_info():
    """Host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def _time_passes(fn, min_seconds, min_passes=3):
    """One warmup call, then timed calls until min_seconds of work; median."""
    fn()
    times, total = [], 0.0
    while len(times) < min_passes or total < min_seconds:
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        times.append(dt)
        total += dt
    return sorted(times)[len(times) // 2], len(times), total


def cpu_baseline(wl, oracle, np, inputs, min_seconds=10.0):
    """The oracle (plain C loops in binary64, OpenMP over output rows) timed on
    the host: the whole decode step (all 197 GEMVs) with every core this
    process may use (the reported value) and with one thread, and a bounded
    sample of the long prefill (the M=4096 gate projection on 64 rows of x)."""
    packed = []
    wbytes = 0
    for t in wl.tensors:
        q, s = oracle.quantize(wl.weight(t), t.bits)
        packed.append((t, q, s))
        wbytes += q.nbytes + s.nbytes
    model, nproc = cpu_info()

    def step(threads):
        for t, q, s in packed:
            oracle.matmul(wl.x_for(t), q, s, t.bits, threads=threads)

    med, n, tot = _time_passes(lambda: step(0), min_seconds)
    med1, n1, tot1 = _time_passes(lambda: step(1), min_seconds / 2)
    lp = inputs.long_prefill()
    gt = lp.tensors[0]
    gq, gs = oracle.quantize(lp.weight(gt), gt.bits)
    gx = lp.x_for(gt)[:64]
    flops = 2 * 64 * gt.N * gt.K
    pm, pn, _ = _time_passes(lambda: oracle.matmul(gx, gq, gs, gt.bits, threads=0), 2.0)
    pm1, pn1, _ = _time_passes(lambda: oracle.matmul(gx, gq, gs, gt.bits, threads=1), 2.0)
    return {
        "value": round(wbytes / med / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.threads_used(),
        "kind": "oracle",
        "sample": f"the full decode step at M=1 ({len(packed)} GEMVs, {wbytes} packed weight bytes): median of "
                  f"{n} passes after 1 warmup ({tot:.1f} s timed), {med:.3f} s per pass, binary64 plain loops",
        "host_cpu": model,
        "nproc": nproc,
        "single_thread": {"value": round(wbytes / med1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "sample": f"the same step, median of {n1} passes, {med1:.3f} s per pass"},
        "prefill_sample": {"workload": "long_prefill gate projection 1024->3072 int4 on 64 of the 4096 rows",
                           "flops": flops,
                           "all_cores_gflops": round(flops / pm / 1e9, 2), "all_cores_s": round(pm, 4),
                           "single_thread_gflops": round(flops / pm1 / 1e9, 2), "single_thread_s": round(pm1, 4),
                           "passes": [pn, pn1]},
    }


def single_gemv_leg(torch, wqa, inputs, np, oracle, reps=512):
    """The single int4 GEMV (M=1, 1024->2048): `reps` launches back to back over
    `reps` distinct packed copies of the weights (604 MB, more than twice the
    256 MB last-level cache), timed with HIP events, directly and as one HIP
    graph; beside it the fixed cost of a launch: the smallest launch of the
    same kernel (M=1, K=32, N=1) timed the same way."""
    wl = inputs.single_gemv()
    t = wl.tensors[0]
    w = wl.weight(t)
    x = torch.from_numpy(wl.x_for(t)).cuda()
    q0, s0 = wqa.pack(torch.from_numpy(w).cuda(), t.bits)
    qs = [q0.clone() for _ in range(reps)]
    ss = [s0.clone() for _ in range(reps)]
    ys = [torch.full((1, t.N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(reps)]
    del q0, s0

    def run():
        for i in range(reps):
            wqa.gemv(x, qs[i], ss[i], t.bits, out=ys[i])

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    direct_ms = timed(run, reps)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.synchronize()
    graph_ms = timed(g.replay, reps)
    # every copy's output equals the oracle within the GEMV bound
    q_ref, s_ref = oracle.quantize(w, t.bits)
    y_ref, B = oracle.matmul(wl.x_for(t), q_ref, s_ref, t.bits)
    first = ys[0].cpu().numpy().astype(np.float64)
    if not (np.all(np.isfinite(first)) and np.all(np.abs(first - y_ref) <= 1e-5 * B)):
        raise SystemExit("bench: single GEMV parity failure")
    for i in range(1, reps):
        if not bool((ys[i] == ys[0]).all()):
            raise SystemExit("bench: single GEMV copies differ")
    # the smallest launch of the same kernel: the fixed cost per launch
    xt = torch.ones((1, 32), dtype=torch.float32, device="cuda")
    qt, st = wqa.pack(torch.ones((1, 32), dtype=torch.float32, device="cuda"), 4)
    yt = torch.empty((1, 1), dtype=torch.float32, device="cuda")
    tiny = lambda: [wqa.gemv(xt, qt, st, 4, out=yt) for _ in range(reps)]
    tiny_ms = timed(tiny, reps)
    gt = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gt, stream=side):
            tiny()
    torch.cuda.synchronize()
    tiny_graph_ms = timed(gt.replay, reps)
    wb = t.weight_bytes
    tb = wl.total_bytes
    del qs, ss, ys
    torch.cuda.empty_cache()
    return {"workload": wl.name, "launches": reps, "distinct_weight_copies": reps,
            "direct": {"us_per_launch": round(direct_ms * 1e3, 3),
                       "weight_gbs": round(wb / (direct_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(tb / (direct_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "graph": {"us_per_launch": round(graph_ms * 1e3, 3),
                      "weight_gbs": round(wb / (graph_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(tb / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "launch_floor": {"what": "M=1, K=32, N=1 GEMV (smallest launch of the same kernel), back to back",
                             "direct_us_per_launch": round(tiny_ms * 1e3, 3),
                             "graph_us_per_launch": round(tiny_graph_ms * 1e3, 3)},
            "weight_bytes": wb, "algorithmic_bytes": tb,
            "note": "ideal at 8 TB/s is 0.149 us per launch; a launch costs more than that by itself"}


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
    lm_w = None
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
        if lm_w is None:
            lm_w = wl.weight(t)
        qr, sr = oracle.quantize(lm_w[ids_h[-1]], t.bits)           # y holds the last lookup
        ref = oracle.embed(np.arange(n), qr, sr, t.K, t.bits)
        if not np.array_equal(y.cpu().numpy().astype(np.float64), ref):
            raise SystemExit(f"bench: embedding lookup of {n} rows differs from the oracle")
        nbytes = n * (t.K * t.bits // 8 + t.K // 32 * 2 + 4 * t.K + 4)
        out[f"embed_{n}"] = {"us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes": nbytes}
    out["table"] = f"int8 lm_head {t.N}x{t.K}, packed; rows bitwise equal to the oracle"
    return out


def mixed_leg(torch, wqa, inputs, np, oracle, steps, warmup, Ms=(1, 2, 4, 8, 16)):
    """Batched decode over the mixed package (attention int8, MLP int4, lm_head
    int8), one grouped launch per step at M = 1, 2, 4, 8 and 16 (M <= 2 on the
    fp32-FMA kernel, M >= 3 on the matrix cores)."""
    out = {}
    for M in Ms:
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


def int5_leg(torch, wqa, inputs, np, oracle, steps, warmup, flush, reps):
    """INT5 (f4): the decode step with every projection packed in int5 (lm_head
    int8) as one grouped launch, and the M=4096 gate projection in int5 through
    the prefill GEMM (cold, like the prefill legs)."""
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
    w = lp.weight(t)
    q, sc = wqa.pack(torch.from_numpy(w).cuda(), 5)
    x = torch.from_numpy(lp.x_for(t)).cuda()
    y = torch.full((t.M, t.N), float("nan"), dtype=torch.float32, device="cuda")
    fn = lambda: wqa.linear(x, q, sc, 5, out=y)
    cold = cold_ms(torch, fn, flush, reps)
    warm = warm_ms(torch, fn, reps)
    rng = np.random.Generator(np.random.PCG64(4545))
    cols = np.sort(rng.choice(t.N, size=64, replace=False))
    rows = np.sort(rng.choice(t.M, size=256, replace=False))
    qr, sr = oracle.quantize(w[cols], 5)
    y_ref, _ = oracle.matmul(lp.x_for(t)[rows], qr, sr, 5)
    yv = y.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
    rel = float(np.linalg.norm(yv - y_ref) / np.linalg.norm(y_ref))
    if not (np.all(np.isfinite(yv)) and rel <= 2e-3):
        raise SystemExit(f"bench: int5 GEMM parity failure: {rel:.3e}")
    tf = 2 * t.M * t.N * t.K / (cold[0] * 1e-3) / 1e12
    out["gemm_gate_m4096"] = {"cold_ms": round(cold[0], 4), "warm_ms": round(warm, 4), "tflops": round(tf, 2),
                              "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                              "parity_rel_frobenius_sample": rel}
    return out


class Flush:
    """Cold-cache protocol: before every cold run a 1 GiB device buffer (4x the
    256 MB last-level cache) is read by a reduction, on the stream of the run
    and outside its HIP-event window. It writes nothing back: a flush that also
    wrote the buffer would leave dirty lines whose write-back then competes with
    the timed call (measured: about 20 us more on the M = 64 lm_head)."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.torch.sum(self.buf, dim=0, keepdim=True, out=self.sink)


def cold_ms(torch, fn, flush, reps):
    """Median over `reps` runs of fn, each right after a cache flush (HIP events
    on the current stream around fn only); also min and max."""
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2], times[0], times[-1]


def warm_ms(torch, fn, reps):
    """The same run repeated back to back on warm caches (HIP events around reps runs)."""
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def prefill_leg(torch, wqa, inputs, np, oracle, flush, reps):
    """Long prefill (M=4096 gate/up/down int4 + int8 lm_head on the last 64
    rows): each wq_linear call timed cold (flush before every run, median of
    `reps`), and warm for comparison; the three MLP GEMMs also as one
    wq_gemm_grouped launch. Each call's output is checked against the oracle on
    sampled rows and columns (relative Frobenius error of the sample)."""
    wl = inputs.long_prefill()
    packed, samples = [], []
    rng = np.random.Generator(np.random.PCG64(4242))
    for t in wl.tensors:
        w = wl.weight(t)
        q, s = wqa.pack(torch.from_numpy(w).cuda(), t.bits)
        cols = np.sort(rng.choice(t.N, size=min(t.N, 64), replace=False))
        samples.append((cols, w[cols].copy()))
        packed.append((q, s))
        del w
    xs = {k: torch.from_numpy(wl.activation(k)).cuda() for k in wl.acts}
    outs = [torch.full((t.M, t.N), float("nan"), dtype=torch.float32, device="cuda") for t in wl.tensors]

    def call(i):
        t = wl.tensors[i]
        return lambda: wqa.linear(xs[t.act][t.act_row0: t.act_row0 + t.M], packed[i][0], packed[i][1], t.bits,
                                  out=outs[i])

    per, warm = [], []
    for i in range(len(wl.tensors)):
        per.append(cold_ms(torch, call(i), flush, reps))
        warm.append(warm_ms(torch, call(i), reps))
    # parity of the timed outputs: 64 sampled columns, 256 sampled rows per call
    worst = 0.0
    for i, t in enumerate(wl.tensors):
        cols, wc = samples[i]
        rows = np.sort(rng.choice(t.M, size=min(t.M, 256), replace=False))
        q, sc = oracle.quantize(wc, t.bits)
        y_ref, _ = oracle.matmul(wl.x_for(t)[rows], q, sc, t.bits)
        y = outs[i].cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
        rel = float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
        if not (np.all(np.isfinite(y)) and rel <= 2e-3):
            raise SystemExit(f"bench: prefill parity failure in {t.name}: {rel:.3e}")
        worst = max(worst, rel)
    gemm_idx = [i for i, t in enumerate(wl.tensors) if t.name != "lm_head"]
    mlp = [wl.tensors[i] for i in gemm_idx]
    mlp_flops = sum(2 * t.M * t.N * t.K for t in mlp)
    mlp_ms = sum(per[i][0] for i in gemm_idx)
    mlp_warm = sum(warm[i] for i in gemm_idx)
    # the same MLP GEMMs (gate, up, down) in one grouped prefill launch
    pkg = wqa.Package([(t.bits, t.N, t.K) for t in mlp])
    for j, t in enumerate(mlp):
        pkg.pack_into(j, torch.from_numpy(wl.weight(t)).cuda())
    gys = [torch.full((t.M, t.N), float("nan"), dtype=torch.float32, device="cuda") for t in mlp]
    gcall = wqa.GroupedCall(pkg, [xs[t.act][t.act_row0: t.act_row0 + t.M] for t in mlp], gys, mlp[0].M,
                            prefill=True)
    g_ms = cold_ms(torch, gcall, flush, reps)
    g_warm = warm_ms(torch, gcall, reps)
    torch.cuda.synchronize()
    # against the per-call outputs (the tile shapes differ: fp32 summation order only)
    g_diff = max(float(torch.linalg.vector_norm(gys[j] - outs[i]) / torch.linalg.vector_norm(outs[i]))
                 for j, i in enumerate(gemm_idx))
    if not g_diff <= 1e-5:
        raise SystemExit(f"bench: grouped MLP outputs differ from wq_linear's: relative {g_diff:.2e}")
    lm = [i for i, t in enumerate(wl.tensors) if t.name == "lm_head"][0]
    lt = wl.tensors[lm]
    lm_bytes = lt.weight_bytes + 4 * lt.M * lt.K + 4 * lt.M * lt.N
    tf = mlp_flops / (mlp_ms * 1e-3) / 1e12
    tfg = mlp_flops / (g_ms[0] * 1e-3) / 1e12
    return {
        "workload": wl.name,
        "protocol": f"cold: a 1 GiB read-only flush before every run, median of {reps}; warm: {reps} runs back "
                    "to back; HIP events around the call only; every call includes its x preparation (a pre-pass kernel, or inside the skinny kernel)",
        "calls": {t.name: {"cold_ms": round(per[i][0], 4), "cold_min_ms": round(per[i][1], 4),
                           "cold_max_ms": round(per[i][2], 4), "warm_ms": round(warm[i], 4),
                           "tflops_cold": round(2 * t.M * t.N * t.K / (per[i][0] * 1e-3) / 1e12, 2)}
                  for i, t in enumerate(wl.tensors)},
        "tflops": round(wl.flops / (sum(p[0] for p in per) * 1e-3) / 1e12, 2),
        "ms_per_step": round(sum(p[0] for p in per), 4),
        "mlp_gemm": {"calls": "gate, up, down at M=4096 (int4), three wq_linear calls, cold",
                     "tflops": round(tf, 2), "ms": round(mlp_ms, 4), "warm_ms": round(mlp_warm, 4),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}},
        "mlp_gemm_grouped": {"calls": "gate, up, down at M=4096 in one wq_gemm_grouped launch, cold",
                             "tflops": round(tfg, 2), "ms": round(g_ms[0], 4), "warm_ms": round(g_warm, 4),
                             "rel_diff_vs_per_call": g_diff, "frac": round(tfg / MFMA_F16_PEAK_TFLOPS, 4)},
        "lm_head_m64": {"cold_ms": round(per[lm][0], 4), "warm_ms": round(warm[lm], 4),
                        "gbs": round(lm_bytes / (per[lm][0] * 1e-3) / 1e9, 1),
                        "hbm_frac": round(lm_bytes / (per[lm][0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "warm_hbm_frac": round(lm_bytes / (warm[lm] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "bytes": lm_bytes},
        "parity_worst_rel_frobenius_sample": worst,
    }


def layer_prefill_leg(torch, wqa, inputs, np, oracle, flush, reps):
    """Prefill through the seven int4 projections of one layer (M = 128 and
    1024): one grouped prefill launch over the layer's tensor table, and the
    seven wq_gemm launches back to back; cold (flush before every run) and warm.
    Outputs of the grouped launch are checked against the oracle on sampled
    rows and columns."""
    out = {}
    rng = np.random.Generator(np.random.PCG64(4343))
    for M in (128, 1024):
        wl = inputs.prefill_layer(M)
        specs = [(t.bits, t.N, t.K) for t in wl.tensors]
        pkg = wqa.Package(specs)
        samples = []
        for i, t in enumerate(wl.tensors):
            w = wl.weight(t)
            pkg.pack_into(i, torch.from_numpy(w).cuda())
            cols = np.sort(rng.choice(t.N, size=64, replace=False))
            samples.append((cols, w[cols].copy()))
        # projections that read one activation in a layer (q, k, v; gate, up) get the same tensor,
        # so the grouped launch prepares it once
        xd = {k: torch.from_numpy(wl.activation(k)).cuda() for k in wl.acts}
        xs = [xd[t.act] for t in wl.tensors]
        ys = [torch.full((M, t.N), float("nan"), dtype=torch.float32, device="cuda") for t in wl.tensors]
        call = wqa.GroupedCall(pkg, xs, ys, M, prefill=True)
        g = cold_ms(torch, call, flush, reps)
        gw = warm_ms(torch, call, reps)
        for i, t in enumerate(wl.tensors):
            cols, wc = samples[i]
            q, sc = oracle.quantize(wc, t.bits)
            y_ref, _ = oracle.matmul(wl.x_for(t), q, sc, t.bits)
            y = ys[i].cpu().numpy()[:, cols].astype(np.float64)
            rel = float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
            if not (np.all(np.isfinite(y)) and rel <= 2e-3):
                raise SystemExit(f"bench: layer prefill parity failure M={M} {t.name}: {rel:.3e}")

        def seq():
            for i, t in enumerate(wl.tensors):
                wqa.gemm(xs[i], pkg.q(i), pkg.scales(i), t.bits, out=ys[i])

        sq = cold_ms(torch, seq, flush, reps)
        sw = warm_ms(torch, seq, reps)
        flops = sum(2 * M * t.N * t.K for t in wl.tensors)
        out[f"m{M}"] = {"grouped_ms": round(g[0], 5), "grouped_warm_ms": round(gw, 5),
                        "grouped_tflops": round(flops / (g[0] * 1e-3) / 1e12, 2),
                        "sequential_ms": round(sq[0], 5), "sequential_warm_ms": round(sw, 5),
                        "sequential_tflops": round(flops / (sq[0] * 1e-3) / 1e12, 2),
                        "workgroups": call.total_tiles}
    out["note"] = ("7 int4 projections (q, k, v, o, gate, up, down) of one layer, 1% outlier rows; "
                   "grouped = wq_gemm_grouped (x preparation + one GEMM launch); sequential = 7 wq_gemm calls; "
                   f"cold = 1 GiB read-only flush before each run, median of {reps}; HIP events")
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

    if args.mixed_only:
        import numpy as np
        import oracle
        if not 1 <= args.mixed_only <= 16:
            print("bench: --mixed-only takes 1 <= M <= 16", file=sys.stderr)
            return 2
        log(f"mixed decode leg at M={args.mixed_only}")
        res = mixed_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup, Ms=(args.mixed_only,))
        print(json.dumps({"decode_step_mixed": res}), flush=True)
        return 0

    if args.prefill_only:
        import numpy as np
        import oracle
        flush = Flush(torch)
        log("prefill leg")
        res = {"prefill": prefill_leg(torch, wqa, inputs, np, oracle, flush, args.prefill_reps)}
        log("layer prefill leg (grouped prefill launch)")
        res["layer_prefill"] = layer_prefill_leg(torch, wqa, inputs, np, oracle, flush, args.prefill_reps)
        print(json.dumps(res), flush=True)
        return 0

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
        log("single GEMV over 512 distinct copies")
        result["single_gemv"] = single_gemv_leg(torch, wqa, inputs, np, oracle)
        log("shared-input fusion (113 GEMVs)")
        result["decode_step_fused"] = fused_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup)
        log("mixed package, batched decode (M = 1, 2, 4, 8, 16)")
        result["decode_step_mixed"] = mixed_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup)
    flush = None
    if not args.decode_only:
        flush = Flush(torch)
        log("int5 decode step and GEMM")
        result["int5"] = int5_leg(torch, wqa, inputs, np, oracle, args.steps, args.warmup, flush, args.prefill_reps)
    if not args.no_prefill and not args.decode_only:
        log("prefill leg")
        result["prefill"] = prefill_leg(torch, wqa, inputs, np, oracle, flush, args.prefill_reps)
        log("layer prefill leg (grouped prefill launch)")
        result["layer_prefill"] = layer_prefill_leg(torch, wqa, inputs, np, oracle, flush, args.prefill_reps)
    del flush
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not args.decode_only:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, oracle, np, inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
