#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s and µs/call of the W4A8 skinny GEMM on one MI355X.

Headline workload (one "step"): every linear of a 27B-class decoder, 64 layers
of QKV 5120->7168, O 5120->5120, gate+up 5120->34816 and down 17408->5120,
W4A8 with G = 32 and bf16 activations N(0, 1) -- the whole 64-layer sweep at
M = 1 (plain decode), then the sweep again at M = 8 (a verify pass: one
committed and seven draft rows).  That is 256 GEMM launches per sweep over
13.2 GB of weights, each weight read once per sweep, so no cache holds them.
The weight values of one layer are drawn on the host, repacked once on the
GPU, and cloned into 63 more buffers: 64 distinct addresses, one set of
values.  Activations differ per layer and per linear.

Timing: each (M, linear) pair -- the 64 launches of that linear, one per
layer -- is one HIP graph; a step replays the 8 graphs (M = 1 first) on
torch's current stream with a HIP event between every two replays, so every
launch of a kernel instance is timed inside the timed region on the stream it
runs on.  The layer-major order (QKV, O, gate+up, down of layer 0, then
layer 1, ...) is timed too, as a check that the order does not matter.

Algorithmic bytes of one call: packed weights + FP32 scales + activations
(2 bytes per bf16) + fp32 output.  Peak: 8 TB/s HBM3E.

The other workloads (per-call sweeps of the 9B-class layer at M = 1..8, the
1024 x 1024 linear, the fused prologues, the W6 / codebook / lm_head formats,
the split-path comparison, expert banks, decode attention and the tree-MTP
planner) are reported beside the headline; the CPU oracle is timed before the
GPU is touched.

Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s & µs/call, W4A8 skinny GEMM at M=1 and M=8 (frac. of peak)"
PEAK_GBPS = 8000.0
GROUP = 32
LAYERS = 64
LAYER_27B = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120), ("down", 5120, 17408)]
SHAPES_9B = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)]
CFG_27B, CFG_9B = 2, 1            # seed recipe: 1000*config + 10*linear + tensor id
WORKLOAD = ("27B-class decoder step: 64 layers x (QKV 5120->7168, O 5120->5120, gate+up 5120->34816, "
            "down 17408->5120), W4A8 G=32, bf16 activations N(0,1); one step = the 64-layer sweep "
            "at M=1, then at M=8")
COPY_PROBE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4_g32_27b_step.md")
# the sources the timed kernels are built from (kernel, launch planning, W4 instances),
# hashed in this order to tie the committed profile summary to them
KERNEL_SOURCES = ("sk_gemm_kernel.h", "sk_gemm.hip", "sk_gemm_w4.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(n: int, k: int, m: int, g: int = GROUP, xbytes: int = 4, wbits: int = 4) -> int:
    return n * k * wbits // 8 + n * (k // g) * 4 + m * k * xbytes + m * n * 4


def source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "gemm_sk_repack_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def committed_profile(key: str):
    """(HBM bytes per launch, rocprofv3 µs per launch) of kernel instance `key` from
    the committed profile summary; (None, None) when that summary was taken on a
    different kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None, None
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != source_hash():
        return None, None
    t = re.search(r"traffic_bytes_per_launch\[" + re.escape(key) + r"\]:\s*([0-9]+)", text)
    d = re.search(r"rocprof_us_per_launch\[" + re.escape(key) + r"\]:\s*([0-9.]+)", text)
    return (int(t.group(1)) if t else None), (float(d.group(1)) if d else None)


# ============================================================================
# CPU baseline: the oracle, single process and split over cores
# ============================================================================

def _oracle_job(job):
    """Seconds the oracle takes for one call on a row slice of its weight.

    job = (prologue, fmt, rows, k, g, m, seed, bf16).  The inputs are drawn
    (untimed) with the workload's distributions; the timed part is the
    prologue (or the bf16 widening), the per-row quantisation and the linear,
    exactly as the oracle computes them for a parity test."""
    import oracle as O
    import synth as S
    pro, fmt, rows, k, g, m, seed, bf16 = job
    _, _, buf = S.make_weight(fmt, rows, k, g, seed, seed + 1)
    cb = S.codebook(seed + 2) if fmt == S.FMT_W4_CODEBOOK else None
    x = S.activations(seed + 3, m, k)
    x2 = S.activations(seed + 4, m, k) if pro == "swiglu" else None
    gam = S.gamma(seed + 5, k) if pro == "rmsnorm" else None
    bits = S.to_bf16_bits(x) if bf16 else None
    t0 = time.perf_counter()
    if pro == "swiglu":
        h = O.prologue_swiglu(x, x2)
    elif pro == "rmsnorm":
        h = O.prologue_rmsnorm(x, gam, 1e-6)
    elif bf16:
        h = O.bf16_to_f32(bits)
    else:
        h = x
    O.reference(fmt, buf, rows, k, g, h, cb)
    return time.perf_counter() - t0


def _time_oracle_call(pool, procs, pro, fmt, n, k, g, m, seed, bf16, rows1, rows_w):
    """µs per call: single process on `rows1` rows, and `procs` workers on
    `rows_w` rows each (the slowest worker sets the time); both scaled to N rows."""
    rows1 = min(n, rows1)
    t1 = _oracle_job((pro, fmt, rows1, k, g, m, seed, bf16))
    rows_w = min(rows_w, -(-n // procs))
    ts = pool.map(_oracle_job, [(pro, fmt, rows_w, k, g, m, seed + 97 * (i + 1), bf16)
                                for i in range(procs)])
    return t1 * 1e6 * n / rows1, max(ts) * 1e6 * n / (rows_w * procs), rows1, rows_w


def cpu_baselines(procs: int):
    """The oracle on the host cores (no GPU involved).

    Headline sample: one 27B-class layer (its 4 linears at M = 1 and at M = 8,
    bf16 activations), in one process and split over `procs` worker processes;
    the 64-layer step time is 64 x the layer.  Table: configs 0, 1, 3 and 4 at
    M = 1 and M = 8, row-sampled so each call takes a fraction of a second,
    scaled to the full N."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    t_all = time.perf_counter()
    with ctx.Pool(procs) as pool:
        head = {"single": 0.0, "multi": 0.0}
        head_bytes = 0
        for m in (1, 8):
            for li, (name, n, k) in enumerate(LAYER_27B):
                seed = 900000 + 1000 * li + m
                us1, usp, _, _ = _time_oracle_call(pool, procs, "none", 0, n, k, GROUP, m, seed, True,
                                                   n, -(-n // procs))
                head["single"] += us1
                head["multi"] += usp
                head_bytes += alg_bytes(n, k, m, xbytes=2)
        calls = [(0, "1024x1024", "none", 0, 1024, 1024, 32, 4),
                 *[(1, nm, "none", 0, n, k, 32, 4) for nm, n, k in SHAPES_9B],
                 (3, "rmsnorm+qkv", "rmsnorm", 0, 6144, 4096, 32, 4),
                 (3, "swiglu+down", "swiglu", 0, 4096, 12288, 32, 4),
                 (4, "w6_g64", "none", 2, 12288, 4096, 64, 4),
                 (4, "codebook_g16", "none", 1, 12288, 4096, 16, 4),
                 (4, "lm_head", "none", 0, 151936, 4096, 32, 4)]
        table = []
        for cfg, label, pro, fmt, n, k, g, xb in calls:
            cap = max(64, 2048 * 4096 // k)
            for m in (1, 8):
                us1, usp, r1, rw = _time_oracle_call(pool, procs, pro, fmt, n, k, g, m,
                                                     800000 + 1000 * cfg + 10 * len(table), False, cap, cap)
                b = alg_bytes(n, k, m, g, xbytes=xb, wbits=6 if fmt == 2 else 4) + (64 if fmt == 1 else 0)
                b += (k * 4 if pro == "rmsnorm" else m * k * 4 if pro == "swiglu" else 0)
                table.append({"config": cfg, "call": label, "n": n, "k": k, "g": g, "m": m,
                              "single_us": round(us1, 1), "single_GBps": round(b / us1 / 1e3, 4),
                              "multi_us": round(usp, 1), "multi_GBps": round(b / usp / 1e3, 4),
                              "rows_sampled_single": r1, "rows_sampled_per_worker": rw})
                log(f"cpu oracle cfg {cfg} {label:12s} M={m}: {us1 / 1e3:9.1f} ms single, "
                    f"{usp / 1e3:8.1f} ms on {procs} processes")
    elapsed = time.perf_counter() - t_all
    cpu_model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    multi_gbps = head_bytes / head["multi"] / 1e3
    single_gbps = head_bytes / head["single"] / 1e3
    log(f"cpu oracle 27B layer (M=1 + M=8): {head['single'] / 1e3:.0f} ms single, "
        f"{head['multi'] / 1e3:.0f} ms on {procs} processes; {elapsed:.1f} s in all")
    baseline = {
        "value": round(multi_gbps, 4), "unit": "GB/s", "cores": procs, "kind": "oracle",
        "sample": (f"one 27B-class layer (QKV, O, gate+up, down) at M=1 and at M=8 with bf16 "
                   f"activations through the numpy oracle, N split over {procs} worker processes "
                   f"(one thread each); the 64-layer step is 64 x that layer. Host: {cpu_model}, "
                   f"{len(os.sched_getaffinity(0))} cores visible"),
        "ms_per_step_extrapolated": round(LAYERS * head["multi"] / 1e3, 1),
        "single_process": {"value": round(single_gbps, 4), "unit": "GB/s", "cores": 1,
                           "ms_per_step_extrapolated": round(LAYERS * head["single"] / 1e3, 1),
                           "sample": "the same layer in one process"},
    }
    return baseline, {"cores": procs, "cpu": cpu_model, "per_call": table,
                      "note": ("the oracle on row samples of each call, scaled to the full N: "
                               "single process, and split over worker processes (the slowest "
                               "worker sets the time)")}


# ============================================================================
# GPU helpers
# ============================================================================

def graph_of(torch, fn):
    """fn() captured in a HIP graph, after one eager call (a call that grows the
    library's default workspace must not be captured), replayed once untimed."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def time_replays(torch, stream, g, reps=3):
    """Milliseconds per replay of g (median of `reps`), HIP events on `stream`."""
    t = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b))
    return float(np.median(t)), t


def time_graph(torch, stream, fn, calls, reps=3):
    """µs per call of `calls` invocations of fn(i) captured in one HIP graph."""
    g = graph_of(torch, lambda: [fn(i) for i in range(calls)])
    ms, _ = time_replays(torch, stream, g, reps)
    return ms * 1e3 / calls


def probe_us(torch, sk, stream, bufs, out):
    """The streaming-read probe over `bufs` (one launch per buffer): the best µs
    per buffer over a few launch shapes, as the ceiling a kernel reading those
    bytes can reach."""
    best = None
    for grid in (256, 512, 1024, 2048):
        for threads in (256, 1024):
            us = time_graph(torch, stream, lambda i: sk.stream_read(bufs[i % len(bufs)], grid, threads, out),
                            len(bufs))
            best = us if best is None else min(best, us)
    return best


def instance_of(sk, n, k, m, xt):
    """(key, template-argument pattern) of the kernel instance a W4 G=32 call runs."""
    p = sk.gemm_plan(n, k, GROUP, sk.SK_W4_SYM, m)
    dot4, wide, pipe4 = m == 1, bool(p["wide"]), p["pipe"] == 4
    key = f"{'dot4' if dot4 else 'mfma'}_{'wide' if wide else 'narrow'}{'_pipe4' if pipe4 else ''}"
    # the last template argument: 4 for the 4-slot pipeline instances, else 0
    pat = (r"gemm_kernel<0, 0, " + str(xt) + r", \d+, " + ("true" if dot4 else "false")
           + r", false, false, " + ("true" if wide else "false") + (", 4>" if pipe4 else ", 0>"))
    return key, pat


# ============================================================================
# headline: the 27B-class 64-layer step
# ============================================================================

def setup_27b(torch, sk, S, host27, dev):
    layers, xs, ys = {}, {}, {}
    for name, n, k in LAYER_27B:
        base = sk.QuantWeight(torch.from_numpy(host27[name]).to(dev), n, k, GROUP, sk.SK_W4_SYM)
        sk.sk_repack_w4a8(base)
        copies = [base]
        for _ in range(LAYERS - 1):
            c = sk.QuantWeight(base.data.clone(), n, k, GROUP, sk.SK_W4_SYM)
            c.desc.layout = sk.SK_LAYOUT_STREAM          # bytes cloned from a repacked weight
            copies.append(c)
        layers[name] = copies
    for li, (name, n, k) in enumerate(LAYER_27B):
        for m in (1, 8):
            ys[(name, m)] = torch.empty((m, n), dtype=torch.float32, device=dev)
            for L in range(LAYERS):
                h = S.activations(1000 * S.seed_of(CFG_27B, li, S.TENSOR_X) + 8 * L + m, m, k)
                bits = S.to_bf16_bits(h)
                xs[(L, name, m)] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    torch.cuda.synchronize()
    return layers, xs, ys


def run_headline(torch, sk, S, host27, args, stream, dev):
    t0 = time.time()
    layers, xs, ys = setup_27b(torch, sk, S, host27, dev)
    wbytes = sum(w.data.numel() for c in layers.values() for w in c)
    log(f"27B step setup {time.time() - t0:.1f}s: {LAYERS} layers, {wbytes / 1e9:.3f} GB of weights")

    def sweep(m, name):
        for L in range(LAYERS):
            sk.sk_gemm_w4a8(layers[name][L], xs[(L, name, m)], y=ys[(name, m)])

    order = [(m, name) for m in (1, 8) for name, _, _ in LAYER_27B]
    for _ in range(args.warmup):
        for m, name in order:
            sweep(m, name)
    torch.cuda.synchronize()
    graphs = {key: graph_of(torch, lambda key=key: sweep(*key)) for key in order}

    # ---------------- timed region ----------------
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for j, key in enumerate(order):
            graphs[key].replay()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize()
    elapsed_ms = ev[0][0].elapsed_time(ev[-1][-1])
    group_ms = {key: [ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(args.steps)]
                for j, key in enumerate(order)}

    shape = {name: (n, k) for name, n, k in LAYER_27B}
    bytes_of = {(m, name): alg_bytes(*shape[name], m, xbytes=2) for m, name in order}
    step_bytes = LAYERS * sum(bytes_of.values())
    ms_per_step = elapsed_ms / args.steps
    value = step_bytes * args.steps / (elapsed_ms * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {elapsed_ms:.2f} ms, {ms_per_step:.3f} ms/step, {value:.0f} GB/s")

    # ---------------- per linear, per sweep ----------------
    probe_out = torch.zeros(4, dtype=torch.int32, device=dev)
    probes = {name: probe_us(torch, sk, stream, [w.data for w in layers[name]], probe_out)
              for name, _, _ in LAYER_27B}
    per, sweeps = [], {}
    for m in (1, 8):
        us_sweep = 0.0
        for name, n, k in LAYER_27B:
            ms = group_ms[(m, name)]
            us = float(np.median(ms)) * 1e3 / LAYERS
            us_sweep += us
            b = bytes_of[(m, name)]
            per.append({"linear": name, "n": n, "k": k, "m": m, "us_per_call": round(us, 3),
                        "us_p10": round(float(np.percentile(ms, 10)) * 1e3 / LAYERS, 3),
                        "us_p90": round(float(np.percentile(ms, 90)) * 1e3 / LAYERS, 3),
                        "GBps": round(b / us / 1e3, 1), "frac_peak": round(b / us / 1e3 / PEAK_GBPS, 4),
                        "probe_us": round(probes[name], 3), "frac_of_probe": round(probes[name] / us, 4)})
            log(f"27B {name:8s} M={m}: {us:8.3f} us/call {per[-1]['GBps']:7.1f} GB/s "
                f"({100 * per[-1]['frac_peak']:.1f}% of peak, {100 * per[-1]['frac_of_probe']:.0f}% of the probe)")
        b = LAYERS * sum(bytes_of[(m, name)] for name, _, _ in LAYER_27B)
        sweeps[m] = {"us_per_sweep": round(LAYERS * us_sweep, 1), "GBps": round(b / (LAYERS * us_sweep) / 1e3, 1),
                     "frac_peak": round(b / (LAYERS * us_sweep) / 1e3 / PEAK_GBPS, 4), "bytes": b}
    for p in per:
        if p["m"] == 8:
            p1 = next(q for q in per if q["m"] == 1 and q["linear"] == p["linear"])
            p["m8_over_m1"] = round(p["us_per_call"] / p1["us_per_call"], 4)

    # ---------------- the same sweeps in layer order ----------------
    layer_major = {}
    for m in (1, 8):
        g = graph_of(torch, lambda m=m: [sk.sk_gemm_w4a8(layers[name][L], xs[(L, name, m)], y=ys[(name, m)])
                                         for L in range(LAYERS) for name, _, _ in LAYER_27B])
        ms, _ = time_replays(torch, stream, g, 5)
        layer_major[m] = {"us_per_sweep": round(ms * 1e3, 1),
                          "vs_linear_major": round(ms * 1e3 / sweeps[m]["us_per_sweep"], 4)}
        log(f"27B layer-major sweep M={m}: {ms * 1e3:.1f} us ({layer_major[m]['vs_linear_major']} x linear-major)")
        del g

    # ---------------- per kernel instance: the roofline ----------------
    inst = {}
    for m, name in order:
        key, pat = instance_of(sk, *shape[name], m, 1)
        d = inst.setdefault(key, {"kernel_pattern": pat, "launches_per_step": 0, "us_per_step": 0.0,
                                  "bytes_per_step": 0, "linears": []})
        d["launches_per_step"] += LAYERS
        d["us_per_step"] += float(np.median(group_ms[(m, name)])) * 1e3
        d["bytes_per_step"] += LAYERS * bytes_of[(m, name)]
        d["linears"].append(f"{name} M={m}")
    for key, d in inst.items():
        d["us_per_launch"] = round(d["us_per_step"] / d["launches_per_step"], 3)
        d["bytes_per_launch"] = d["bytes_per_step"] // d["launches_per_step"]
        d["GBps"] = round(d["bytes_per_launch"] / d["us_per_launch"] / 1e3, 1)
        d["traffic_bytes_per_launch"], d["rocprof_us_per_launch"] = committed_profile(key)
        d["us_per_step"] = round(d["us_per_step"], 1)
    dom = max(inst, key=lambda kk: inst[kk]["us_per_step"])
    d = inst[dom]
    achieved = d["bytes_per_launch"] / d["us_per_launch"] / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": d["traffic_bytes_per_launch"],
                "kernel": f"{d['kernel_pattern']} ({dom}: {', '.join(d['linears'])})",
                "bytes_per_launch": d["bytes_per_launch"], "us_per_launch": d["us_per_launch"],
                "launches_per_step": d["launches_per_step"],
                "rocprof_us_per_launch": d["rocprof_us_per_launch"]}
    log(f"dominant kernel {dom}: {d['us_per_launch']} us/launch, {achieved:.0f} GB/s "
        f"({100 * achieved / PEAK_GBPS:.1f}% of peak)")
    res = {"value": value, "ms_per_step": ms_per_step, "step_bytes": step_bytes, "weight_bytes": wbytes,
           "per": per, "sweeps": sweeps, "layer_major": layer_major, "instances": inst,
           "roofline": roofline}
    del graphs, layers, xs, ys
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def profile_27b(torch, sk, S, host27, dev, steps):
    """`steps` eager steps of the headline workload, no timing: the run that
    rocprofv3 counter passes observe."""
    layers, xs, ys = setup_27b(torch, sk, S, host27, dev)
    for _ in range(steps):
        for m in (1, 8):
            for name, _, _ in LAYER_27B:
                for L in range(LAYERS):
                    sk.sk_gemm_w4a8(layers[name][L], xs[(L, name, m)], y=ys[(name, m)])
    torch.cuda.synchronize()
    log(f"profile run: {steps} eager steps of {8 * LAYERS} launches")


# ============================================================================
# the 9B-class layer: per-call sweep over M, split-path comparison
# ============================================================================

def run_9b(torch, sk, S, dev, stream, copies, ms_list):
    """Per-call µs of the 9B-class layer's linears (fp32 activations) at each M,
    R rotated weight copies per linear (more than 1 GiB in all), with the
    streaming-read probe on the same buffers."""
    R = copies + copies % 2
    host, weights = {}, {}
    for li, (name, n, k) in enumerate(SHAPES_9B):
        _, _, buf = S.make_weight(S.FMT_W4, n, k, GROUP, S.seed_of(CFG_9B, li, S.TENSOR_W),
                                  S.seed_of(CFG_9B, li, S.TENSOR_S))
        host[name] = buf
        base = sk.QuantWeight(torch.from_numpy(buf).to(dev), n, k, GROUP, sk.SK_W4_SYM)
        sk.sk_repack_w4a8(base)
        cps = [base]
        for _ in range(R - 1):
            c = sk.QuantWeight(base.data.clone(), n, k, GROUP, sk.SK_W4_SYM)
            c.desc.layout = sk.SK_LAYOUT_STREAM
            cps.append(c)
        weights[name] = cps
    xs = {(m, k): torch.from_numpy(S.activations(S.seed_of(CFG_9B, m, S.TENSOR_X) + k, m, k)).to(dev)
          for m in range(1, 9) for k in sorted({k for _, _, k in SHAPES_9B})}
    ys = {(name, m): torch.empty((m, n), dtype=torch.float32, device=dev)
          for name, n, _ in SHAPES_9B for m in range(1, 9)}
    probe_out = torch.zeros(4, dtype=torch.int32, device=dev)
    per = []
    for name, n, k in SHAPES_9B:
        pr = probe_us(torch, sk, stream, [w.data for w in weights[name]], probe_out)
        for m in ms_list:
            g = graph_of(torch, lambda: [sk.sk_gemm_w4a8(weights[name][r % R], xs[(m, k)], y=ys[(name, m)])
                                         for r in range(4 * R)])
            med, t = time_replays(torch, stream, g, 7)
            us = med * 1e3 / (4 * R)
            b = alg_bytes(n, k, m)
            per.append({"linear": name, "n": n, "k": k, "m": m, "us_per_call": round(us, 3),
                        "us_p10": round(float(np.percentile(t, 10)) * 1e3 / (4 * R), 3),
                        "us_p90": round(float(np.percentile(t, 90)) * 1e3 / (4 * R), 3),
                        "GBps": round(b / us / 1e3, 1), "frac_peak": round(b / us / 1e3 / PEAK_GBPS, 4),
                        "probe_us": round(pr, 3), "frac_of_probe": round(pr / us, 4)})
            log(f"9B  {name:8s} M={m}: {us:8.3f} us/call {per[-1]['GBps']:7.1f} GB/s "
                f"({100 * per[-1]['frac_peak']:.1f}% of peak, {100 * per[-1]['frac_of_probe']:.0f}% of the probe)")
    layer = {}
    for m in (1, 8):
        rows = [p for p in per if p["m"] == m]
        if len(rows) == len(SHAPES_9B):
            us = sum(p["us_per_call"] for p in rows)
            b = sum(alg_bytes(p["n"], p["k"], m) for p in rows)
            layer[f"m{m}"] = {"us_per_layer": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    if "m1" in layer and "m8" in layer:
        layer["m8_over_m1"] = round(layer["m8"]["us_per_layer"] / layer["m1"]["us_per_layer"], 4)
    del weights
    return {"workload": ("9B-class decoder layer linears, W4A8 G=32, fp32 activations: QKV 4096->6144, "
                         "O 4096->4096, gate+up 4096->24576, down 12288->4096"),
            "weight_copies_rotated": R, "per_call": per, "layer": layer}, host, xs, R


def time_ablation(torch, sk, stream, host, xs, R, per):
    """The 9B-class layer's calls on the split path: (a) the weight left in the
    canonical layout (codes and scales read from their two regions), quantising
    in the launch; (b) also quantising in a launch of its own, q and sx through
    memory.  µs per call from graphs over R rotated canonical copies."""
    dev = torch.device("cuda:0")
    rows = []
    tot = {"fused": 0.0, "canonical": 0.0, "split": 0.0}
    for name, n, k in SHAPES_9B:
        base = torch.from_numpy(host[name]).to(dev)
        cps = [sk.QuantWeight(base if i == 0 else base.clone(), n, k, GROUP, sk.SK_W4_SYM)
               for i in range(R)]
        for m in (1, 8):
            x = xs[(m, k)]
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            q = torch.empty((m, k), dtype=torch.int8, device=dev)
            sx = torch.empty((m,), dtype=torch.float32, device=dev)
            us_can = time_graph(torch, stream, lambda i: sk.sk_gemm_w4a8_canonical(cps[i % R], x, y=y),
                                4 * R)

            def split(i):
                sk.sk_quantize_rows(x, q=q, sx=sx)
                sk.sk_gemm_w4a8_canonical_q(cps[i % R], q, sx, y=y)
            us_split = time_graph(torch, stream, split, 4 * R)
            us_fused = next(p["us_per_call"] for p in per if p["linear"] == name and p["m"] == m)
            b = alg_bytes(n, k, m)
            rows.append({"linear": name, "m": m, "fused_us": round(us_fused, 3),
                         "canonical_us": round(us_can, 3), "split_us": round(us_split, 3),
                         "fused_GBps": round(b / us_fused / 1e3, 1),
                         "split_GBps": round(b / us_split / 1e3, 1)})
            tot["fused"] += us_fused
            tot["canonical"] += us_can
            tot["split"] += us_split
            log(f"split path {name:8s} M={m}: fused {us_fused:7.3f}  canonical {us_can:7.3f}  "
                f"canonical + separate quantisation {us_split:7.3f} us/call")
        del cps, base
    return {"what": ("the 9B-class layer's 8 calls on (a) the weight in the canonical layout, "
                     "quantising in the launch, and (b) that plus quantisation as its own launch "
                     "(q, sx through memory), against the fused stream-layout path"),
            "step_us": {kk: round(v, 3) for kk, v in tot.items()},
            "speedup_of_fused": {"over_canonical": round(tot["canonical"] / tot["fused"], 4),
                                 "over_split": round(tot["split"] / tot["fused"], 4)},
            "per_call": rows}


# ============================================================================
# other workloads
# ============================================================================

def time_experts(torch, sk, S, stream):
    """Expert-bank workload (synthetic): a W4A8 G=32 bank of 32 experts x 2048
    rows at K = 4096 (168 MB), 7 rotated copies (1.2 GB); M = 1 with 2 listed
    experts and M = 8 with 8, a fresh device list per call.  One sk_gemm_experts
    launch against one sk_gemm_w4a8 launch per listed expert."""
    dev = torch.device("cuda:0")
    E, rows, k, g, R = 32, 2048, 4096, 32, 7
    _, _, buf = S.make_weight(0, E * rows, k, g, S.seed_of(5, 0, S.TENSOR_W), S.seed_of(5, 0, S.TENSOR_S))
    base = sk.QuantWeight(torch.from_numpy(buf).to(dev), E * rows, k, g, sk.SK_W4_SYM)
    sk.sk_repack_w4a8(base)
    banks = [base]
    for _ in range(R - 1):
        c = sk.QuantWeight(base.data.clone(), E * rows, k, g, sk.SK_W4_SYM)
        c.desc.layout = sk.SK_LAYOUT_STREAM
        banks.append(c)
    eb = sk.weight_bytes(sk.SK_W4_SYM, rows, k, g)       # one expert's bytes, contiguous in the bank

    def view(b, e):
        v = sk.QuantWeight(banks[b].data[e * eb:(e + 1) * eb], rows, k, g, sk.SK_W4_SYM)
        v.desc.layout = sk.SK_LAYOUT_STREAM
        return v
    views = [[view(b, e) for e in range(E)] for b in range(R)]
    rng = np.random.default_rng(S.seed_of(5, 0, 9))
    out = []
    for m, nl in ((1, 2), (8, 8)):
        lists = [sorted(rng.choice(E, nl, replace=False).tolist()) for _ in range(16)]
        dlists = [torch.tensor(lst, dtype=torch.int32, device=dev) for lst in lists]
        x = torch.from_numpy(S.activations(S.seed_of(5, m, S.TENSOR_X), m, k)).to(dev)
        y = torch.empty((m, nl * rows), dtype=torch.float32, device=dev)
        ys = [torch.empty((m, rows), dtype=torch.float32, device=dev) for _ in range(nl)]
        us_bank = time_graph(torch, stream,
                             lambda i: sk.sk_gemm_experts(banks[i % R], rows, dlists[i % 16], x, y=y), 4 * R)

        def separate(i):
            for j, e in enumerate(lists[i % 16]):
                sk.sk_gemm_w4a8(views[i % R][e], x, y=ys[j])
        us_sep = time_graph(torch, stream, separate, 4 * R)
        b = alg_bytes(nl * rows, k, m)
        out.append({"m": m, "experts_per_call": nl, "us_per_call": round(us_bank, 3),
                    "GBps": round(b / us_bank / 1e3, 1),
                    "separate_launches_us": round(us_sep, 3),
                    "separate_GBps": round(b / us_sep / 1e3, 1)})
        log(f"experts M={m} x{nl}: one launch {us_bank:7.3f} us ({out[-1]['GBps']} GB/s), "
            f"{nl} launches {us_sep:7.3f} us")
    del views, banks, base
    return {"workload": ("synthetic W4A8 G=32 expert bank, 32 experts x 2048 rows, K = 4096, "
                         "7 rotated copies; a fresh device expert list per call"),
            "per_call": out}


def time_attention(torch, sk, S, stream):
    """Grouped-query decode attention of the 9B-class layer (synthetic): Hq 32,
    Hkv 8, head dim 128, bf16 KV cache in the library's tiled layout, prefix L
    in {4096, 16384, 32768}, M = 1 and M = 8 verification rows.  Rotated cache
    copies (>= 1 GiB in total) so every call streams from HBM; µs per call
    from graphs; GB/s over the algorithmic bytes (the prefix's K and V, q, O)."""
    dev = torch.device("cuda:0")
    hq, hkv, d = 32, 8, 128
    out = []
    for length in (4096, 16384, 32768):
        _, kb, vb = S.attention_inputs(S.seed_of(6, 0, 0), 1, hq, hkv, length)
        base = torch.from_numpy(sk.sk_kv_pack_host(kb, vb, hkv, length, length)).to(dev)
        R = max(2, (1 << 30) // base.numel())
        caches = [base] + [base.clone() for _ in range(R - 1)]
        kv_bytes = 2 * hkv * length * d * 2
        for m in (1, 8):
            qb, _, _ = S.attention_inputs(S.seed_of(6, m, 0), m, hq, hkv, 1)
            q = torch.from_numpy(qb.view(np.int16)).to(dev)
            o = torch.empty((m, hq, d), dtype=torch.float32, device=dev)
            us = time_graph(torch, stream,
                            lambda i: sk.sk_decode_attention(q, hkv, caches[i % R], length, length, out=o),
                            4 * R)
            b = kv_bytes + m * hq * d * (2 + 4)
            splits, bps = sk.attention_plan(m, hq, hkv, length)
            gbps = b / us / 1e3
            out.append({"L": length, "m": m, "us_per_call": round(us, 3),
                        "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4),
                        "ranges_per_head": splits, "blocks_per_range": bps})
            log(f"attention L={length} M={m}: {us:7.3f} us ({out[-1]['GBps']} GB/s), "
                f"{splits} ranges x {bps} blocks per head")
        del caches, base
    return {"workload": ("synthetic 9B-class GQA decode attention: Hq 32, Hkv 8, head dim 128, "
                         "bf16 KV cache (tiled), causal verification rows; rotated cache copies"),
            "per_call": out}


def plan_mtp(sk, plain_ms: float, verify_ms: float, draft_ms: float):
    """The library's tree-MTP planner on synthetic acceptance statistics, with
    this run's measured costs: verify = the 64-layer sweep of the 27B-class
    linears at M = 8, draft = one layer's linears at M = 1, plain decoding =
    the sweep at M = 1.  Attention and the rest of the layer are left out on
    every side.  Reports the layout the planner settles on, the mean tokens per
    step and the rate against plain decoding."""
    rng = np.random.default_rng(0)
    regimes = {
        "code-like": [0.04, 0.86, 0.06, 0.02, 0.01, 0.005, 0.003, 0.002],
        "creative-like": [0.15, 0.35, 0.25, 0.13, 0.05, 0.03, 0.02, 0.02],
    }
    out = []
    for name, probs in regimes.items():
        pl = sk.MtpPlanner()
        w = [1] * 7
        toks = []
        for step in range(640):
            ranks_all = [int(rng.choice(8, p=probs)) for _ in range(7)]
            acc, obs = sk.mtp_accept(w, ranks_all[:len(w)])
            if step >= 320:
                toks.append((1 + acc, len(w)))
            w = pl.observe(ranks_all[:obs], verify_ms, draft_ms)
        tok = float(np.mean([t for t, _ in toks]))
        cost = float(np.mean([verify_ms + d * draft_ms for _, d in toks]))
        chain_tok = sum(probs[1] ** i for i in range(8))
        out.append({"regime": name, "layout": w, "tokens_per_step": round(tok, 3),
                    "speedup_vs_plain_decode": round((tok / cost) / (1.0 / plain_ms), 3),
                    "chain_of_7_expected_tokens": round(chain_tok, 3)})
        log(f"mtp {name}: layout {w}, {tok:.2f} tokens/step, "
            f"x{out[-1]['speedup_vs_plain_decode']} vs plain decoding")
    return {"verify_ms": round(verify_ms, 4), "draft_ms": round(draft_ms, 4), "plain_ms": round(plain_ms, 4),
            "note": ("synthetic rank statistics; costs from this run's 27B-class linears "
                     "(the 64-layer sweep at M = 8 to verify, one layer at M = 1 to draft)"),
            "regimes": out}


def time_variants(torch, sk, S, dev, stream):
    """The single 1024 x 1024 linear, the fused prologues at hidden 4096, the
    W6 / codebook / lm_head formats at K = 4096, and the 27B-class lm_head
    (5120 -> 151936, bf16 activations)."""
    rows = []

    def weight_copies(fmt, n, k, g, cfg, li):
        _, _, buf = S.make_weight(fmt, n, k, g, S.seed_of(cfg, li, S.TENSOR_W),
                                  S.seed_of(cfg, li, S.TENSOR_S))
        cb = (torch.from_numpy(S.codebook(S.seed_of(cfg, li, S.TENSOR_CB))).to(dev)
              if fmt == sk.SK_W4_CODEBOOK else None)
        base = sk.QuantWeight(torch.from_numpy(buf).to(dev), n, k, g, fmt, cb)
        sk.sk_repack_w4a8(base)
        copies = [base]
        # more than 1 GiB of distinct weight bytes between two reads of one copy
        for _ in range(max(1, -(-(5 << 28) // buf.nbytes)) - 1):
            c = sk.QuantWeight(base.data.clone(), n, k, g, fmt, cb)
            c.desc.layout = sk.SK_LAYOUT_STREAM
            copies.append(c)
        return copies, buf.nbytes

    def record(group, name, n, k, g, fmt, m, us, nbytes, extra=0, xbytes=4):
        alg = nbytes + (64 if fmt == sk.SK_W4_CODEBOOK else 0) + m * k * xbytes + m * n * 4 + extra
        rows.append({"group": group, "linear": name, "n": n, "k": k, "g": g,
                     "format": {0: "W4", 1: "W4 codebook", 2: "W6"}[fmt], "m": m,
                     "us_per_call": round(us, 3), "GBps": round(alg / us / 1e3, 1),
                     "frac_peak": round(alg / us / 1e3 / PEAK_GBPS, 4)})
        log(f"{group:10s} {name:12s} M={m}: {us:8.3f} us/call {rows[-1]['GBps']:7.1f} GB/s")

    # the single small linear (N = K = 1024, 0.66 MB): latency-bound and
    # cache-resident, so reported in µs (its GB/s is not a bandwidth figure)
    cps, nb = weight_copies(sk.SK_W4_SYM, 1024, 1024, 32, 0, 0)
    for m in (1, 8):
        x = torch.from_numpy(S.activations(S.seed_of(0, 0, S.TENSOR_X), m, 1024)).to(dev)
        y = torch.empty((m, 1024), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_w4a8(cps[i % len(cps)], x, y=y), 4 * len(cps))
        record("small", "1024x1024", 1024, 1024, 32, 0, m, us, nb)
    del cps

    # fused prologues at hidden 4096, beside the same calls split into launches:
    # (a) the prologue launch writing h, then the GEMM quantising in its launch;
    # (b) the prologue launch, the quantisation launch, then the GEMM on the
    #     weight in the canonical layout
    def split_times(cps, n, k, m, prologue):
        can = [sk.QuantWeight(c.data.clone(), n, k, 32, sk.SK_W4_SYM) for c in cps]
        for c in can:                                     # canonical bytes of the same weight
            c.desc.layout = sk.SK_LAYOUT_STREAM
            sk.sk_unrepack_w4a8(c)
        h = torch.empty((m, k), dtype=torch.float32, device=dev)
        q = torch.empty((m, k), dtype=torch.int8, device=dev)
        sx = torch.empty((m,), dtype=torch.float32, device=dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        R = len(cps)

        def a(i):
            prologue(h)
            sk.sk_gemm_w4a8(cps[i % R], h, y=y)

        def b(i):
            prologue(h)
            sk.sk_quantize_rows(h, q=q, sx=sx)
            sk.sk_gemm_w4a8_canonical_q(can[i % R], q, sx, y=y)
        us_a = time_graph(torch, stream, a, 4 * R)
        us_b = time_graph(torch, stream, b, 4 * R)
        del can
        return us_a, us_b

    cps, nb = weight_copies(sk.SK_W4_SYM, 6144, 4096, 32, 3, 0)
    gam = torch.from_numpy(S.gamma(S.seed_of(3, 0, S.TENSOR_GAMMA), 4096)).to(dev)
    for m in (1, 3, 8):
        x = torch.from_numpy(S.activations(S.seed_of(3, 0, S.TENSOR_X), m, 4096)).to(dev)
        y = torch.empty((m, 6144), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_fused_rmsnorm(
            cps[i % len(cps)], x, gam, 1e-6, y=y), 4 * len(cps))
        record("fused", "rmsnorm+qkv", 6144, 4096, 32, 0, m, us, nb, extra=4096 * 4)
        us_a, us_b = split_times(cps, 6144, 4096, m, lambda h: sk.sk_prologue_rmsnorm(x, gam, 1e-6, h=h))
        rows[-1].update({"split_prologue_us": round(us_a, 3), "split_prologue_quant_canonical_us": round(us_b, 3)})
        log(f"{'':10s} {'':12s} split: prologue launch + GEMM {us_a:8.3f} us; "
            f"+ quantisation launch + canonical GEMM {us_b:8.3f} us")
    del cps
    cps, nb = weight_copies(sk.SK_W4_SYM, 4096, 12288, 32, 3, 1)
    for m in (1, 3, 8):
        gu = torch.from_numpy(np.concatenate(
            [S.activations(S.seed_of(3, 1, S.TENSOR_GATE), m, 12288),
             S.activations(S.seed_of(3, 1, S.TENSOR_UP), m, 12288)], axis=1)).to(dev)
        y = torch.empty((m, 4096), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_fused_swiglu(
            cps[i % len(cps)], gu[:, :12288], gu[:, 12288:], y=y), 4 * len(cps))
        record("fused", "swiglu+down", 4096, 12288, 32, 0, m, us, nb, extra=m * 12288 * 4)
        us_a, us_b = split_times(cps, 4096, 12288, m,
                                 lambda h: sk.sk_prologue_swiglu(gu[:, :12288], gu[:, 12288:], h=h))
        rows[-1].update({"split_prologue_us": round(us_a, 3), "split_prologue_quant_canonical_us": round(us_b, 3)})
        log(f"{'':10s} {'':12s} split: prologue launch + GEMM {us_a:8.3f} us; "
            f"+ quantisation launch + canonical GEMM {us_b:8.3f} us")
    del cps
    # formats at K = 4096
    for li, (name, fmt, n, g) in enumerate([("w6_g64", sk.SK_W6_SYM, 12288, 64),
                                            ("codebook_g16", sk.SK_W4_CODEBOOK, 12288, 16),
                                            ("lm_head", sk.SK_W4_SYM, 151936, 32)]):
        cps, nb = weight_copies(fmt, n, 4096, g, 4, li)
        for m in (1, 8):
            x = torch.from_numpy(S.activations(S.seed_of(4, li, S.TENSOR_X), m, 4096)).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            fn = sk.sk_gemm_w6a8 if fmt == sk.SK_W6_SYM else sk.sk_gemm_w4a8
            us = time_graph(torch, stream, lambda i: fn(cps[i % len(cps)], x, y=y), max(8, 2 * len(cps)))
            record("formats", name, n, 4096, g, fmt, m, us, nb)
        del cps
    # the 27B-class lm_head, reported beside the step (not part of it)
    cps, nb = weight_copies(sk.SK_W4_SYM, 151936, 5120, 32, 2, 4)
    for m in (1, 8):
        bits = S.to_bf16_bits(S.activations(S.seed_of(2, 4, S.TENSOR_X), m, 5120))
        x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((m, 151936), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_w4a8(cps[i % len(cps)], x, y=y), max(8, 2 * len(cps)))
        record("27b", "lm_head", 151936, 5120, 32, 0, m, us, nb, xbytes=2)
    del cps
    return rows


# ============================================================================
# profile summary (reads rocprofv3 CSV output; no GPU)
# ============================================================================

PROFILE_COMMANDS = {
    "trace": ("rocprofv3 --kernel-trace --stats -d $OUT/trace -o trace --output-format csv -- "
              "python3 $R/bench.py --steps 10 --warmup 2 --headline-only"),
    "FETCH_SIZE": ("rocprofv3 --pmc FETCH_SIZE -d $OUT/FETCH_SIZE -o pmc --output-format csv -- "
                   "python3 $R/bench.py --profile-steps 1"),
    "WRITE_SIZE": ("rocprofv3 --pmc WRITE_SIZE -d $OUT/WRITE_SIZE -o pmc --output-format csv -- "
                   "python3 $R/bench.py --profile-steps 1"),
    "copy_FETCH_SIZE": ("rocprofv3 --pmc FETCH_SIZE -d $OUT/copy_FETCH_SIZE -o pmc --output-format csv -- "
                        "python3 $R/bench.py --copy-probe"),
    "copy_WRITE_SIZE": ("rocprofv3 --pmc WRITE_SIZE -d $OUT/copy_WRITE_SIZE -o pmc --output-format csv -- "
                        "python3 $R/bench.py --copy-probe"),
}


def _csv_rows(path):
    import csv
    files = sorted(glob.glob(path))
    if not files:
        raise SystemExit(f"no file matches {path}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def summarize_profiles(out_dir: str) -> str:
    """Markdown summary of the rocprofv3 runs under out_dir (PROFILE_COMMANDS)
    and of the bench line the traced run printed (out_dir/bench.json)."""
    bench = json.loads(open(os.path.join(out_dir, "bench.json")).read().strip().splitlines()[-1])
    inst = bench["instances"]
    trace = _csv_rows(os.path.join(out_dir, "trace", "*kernel_trace.csv"))
    dur = {}
    for r in trace:
        dur.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def match(pat, names):
        got = [nm for nm in names if re.search(pat, nm)]
        if len(got) != 1:
            raise SystemExit(f"{pat}: {len(got)} kernels match")
        return got[0]

    def counters(sub):
        per = {}
        for r in _csv_rows(os.path.join(out_dir, sub, "*counter_collection.csv")):
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return per

    fetch, write = counters("FETCH_SIZE"), counters("WRITE_SIZE")
    cf, cw = counters("copy_FETCH_SIZE"), counters("copy_WRITE_SIZE")
    copy_name = match(r"copyBuffer", cf.keys())
    copy_kib = COPY_PROBE_BYTES / 1024
    f_scale = copy_kib / float(np.mean(cf[copy_name]))
    w_scale = copy_kib / float(np.mean(cw[match(r"copyBuffer", cw.keys())]))

    lines = [
        "# GEMM kernels on the 27B-class 64-layer step: kernel time and HBM traffic", "",
        f"Workload: {WORKLOAD}. MI355X, one GPU.", "",
        "In the commands, R is the repository root and OUT an output directory; each runs",
        "from `/tmp` with `TMPDIR=/tmp`.", "",
        "## Bench line of the traced run", "",
        "    " + PROFILE_COMMANDS["trace"], "",
        f"value {bench['value']} GB/s, {bench['ms_per_step']} ms per step; "
        f"M=1 sweep {bench['m1']['us_per_sweep']} us, M=8 sweep {bench['m8']['us_per_sweep']} us.", "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats, the command above)", "",
        "All dispatches of each kernel in the run: eager warm-up steps, graph replays of the",
        "timed steps and of the layer-major check.  The bench's HIP-event figure is the",
        "timed steps' median per launch, which includes the gap between two launches.", "",
        "| instance | kernel | dispatches | rocprof average us | min us | max us | bench HIP-event us per launch |",
        "|---|---|---|---|---|---|---|",
    ]
    machine = [f"    source_sha256: {source_hash()}"]
    for key, d in sorted(inst.items()):
        nm = match(d["kernel_pattern"], dur.keys())
        v = dur[nm]
        lines.append(f"| {key} | `{nm}` | {len(v)} | {np.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{d['us_per_launch']} |")
        machine.append(f"    rocprof_us_per_launch[{key}]: {np.mean(v):.3f}")
    others = sorted(((sum(v), nm, len(v)) for nm, v in dur.items()
                     if not any(re.search(d["kernel_pattern"], nm) for d in inst.values())), reverse=True)
    lines += ["", "Other kernels in the run (setup: repack, copies, fills):", "",
              "| kernel | dispatches | total us |", "|---|---|---|"]
    lines += [f"| `{nm}` | {c} | {t:.0f} |" for t, nm, c in others[:8]]
    lines += ["", "## HBM bytes (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE, separate runs)", "",
              "Commands:", ""]
    lines += ["    " + PROFILE_COMMANDS[k] for k in ("FETCH_SIZE", "WRITE_SIZE", "copy_FETCH_SIZE",
                                                     "copy_WRITE_SIZE")]
    lines += ["", f"Calibration: a device copy of {COPY_PROBE_BYTES >> 20} MiB reads "
              f"{np.mean(cf[copy_name]):.1f} KiB by FETCH_SIZE and writes "
              f"{np.mean(cw[match(r'copyBuffer', cw.keys())]):.1f} KiB by WRITE_SIZE per dispatch, so "
              f"bytes = FETCH_SIZE x {f_scale:.4f} KiB and WRITE_SIZE x {w_scale:.4f} KiB.", "",
              "| instance | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch (scaled) | "
              "algorithmic bytes / launch | ratio |", "|---|---|---|---|---|---|---|"]
    for key, d in sorted(inst.items()):
        fv = fetch[match(d["kernel_pattern"], fetch.keys())]
        wv = write[match(d["kernel_pattern"], write.keys())]
        hbm = int(round((np.mean(fv) * f_scale + np.mean(wv) * w_scale) * 1024))
        lines.append(f"| {key} | {len(fv)} | {np.mean(fv):.1f} | {np.mean(wv):.1f} | {hbm} | "
                     f"{d['bytes_per_launch']} | {hbm / d['bytes_per_launch']:.3f} |")
        machine.append(f"    traffic_bytes_per_launch[{key}]: {hbm}")
    lines += ["", "Per-launch figures average the instance's launches in one step (e.g. the four",
              "linears of every layer at M=8), as the bench's `bytes_per_launch` does.", "",
              "Machine-readable (bench.py reports these only while the kernel sources",
              ", ".join(KERNEL_SOURCES) + " still hash, in that order, to this value):", ""]
    return "\n".join(lines + machine) + "\n"


# ============================================================================
# main
# ============================================================================

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=10, help="rotated weight copies per 9B-class linear")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the 27B-class step: no CPU baseline and no other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-9b", action="store_true", help="skip the 9B-class per-call sweep and the split path")
    ap.add_argument("--no-sweep", action="store_true", help="9B-class calls at M = 1 and 8 only")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the 1024 x 1024 linear, fused prologues, formats and lm_head")
    ap.add_argument("--no-experts", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-mtp", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="worker processes of the split oracle (default: the visible cores, at most 16)")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many eager steps of the 27B-class workload (no graphs, no timing) "
                         "and exit: the workload of the rocprofv3 counter passes")
    ap.add_argument("--profile-attention", type=int, default=0,
                    help="run this many eager decode-attention calls (L = 16384, M = 1 and 8, "
                         "rotated caches) and exit: the workload of its rocprofv3 kernel trace")
    ap.add_argument("--copy-probe", action="store_true",
                    help="copy a 256 MiB device buffer 5 times and exit: the known-size "
                         "kernel that calibrates the HBM byte counters")
    ap.add_argument("--summarize-profiles", metavar="OUT",
                    help="print the markdown summary of the rocprofv3 runs under OUT and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_profiles:
        sys.stdout.write(summarize_profiles(args.summarize_profiles))
        return 0
    if args.gpus != 1:
        print("bench.py measures the skinny GEMM on one GPU; --gpus above 1 is not supported "
              "(the workload runs on a single MI355X)", file=sys.stderr)
        return 2
    if args.headline_only:
        args.no_cpu_baseline = args.no_9b = args.no_variants = args.no_experts = True
        args.no_attention = args.no_mtp = args.no_ablation = True

    import synth as S
    profiling = bool(args.profile_steps or args.profile_attention or args.copy_probe)

    host27 = None
    if not args.profile_attention and not args.copy_probe:
        t0 = time.time()
        host27 = {}
        for li, (name, n, k) in enumerate(LAYER_27B):
            _, _, host27[name] = S.make_weight(S.FMT_W4, n, k, GROUP, S.seed_of(CFG_27B, li, S.TENSOR_W),
                                               S.seed_of(CFG_27B, li, S.TENSOR_S))
        log(f"host layer drawn in {time.time() - t0:.1f}s")

    # the oracle runs before anything touches the GPU: its worker processes are forked
    cpu, cpu_table = None, None
    if not args.no_cpu_baseline and not profiling:
        procs = args.cpu_procs or min(16, len(os.sched_getaffinity(0)))
        cpu, cpu_table = cpu_baselines(procs)

    import torch

    import gemm_sk_repack_amd as sk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 5 copies of {COPY_PROBE_BYTES} bytes")
        return 0
    if args.profile_attention:
        hq, hkv, length = 32, 8, 16384
        _, kb, vb = S.attention_inputs(S.seed_of(6, 0, 0), 1, hq, hkv, length)
        base = torch.from_numpy(sk.sk_kv_pack_host(kb, vb, hkv, length, length)).to(dev)
        caches = [base] + [base.clone() for _ in range(15)]
        for m in (1, 8):
            qb, _, _ = S.attention_inputs(S.seed_of(6, m, 0), m, hq, hkv, 1)
            q = torch.from_numpy(qb.view(np.int16)).to(dev)
            for i in range(args.profile_attention):
                sk.sk_decode_attention(q, hkv, caches[i % 16], length, length)
        torch.cuda.synchronize()
        log(f"profile run: {args.profile_attention} decode-attention calls at M = 1 and at M = 8")
        return 0
    if args.profile_steps:
        profile_27b(torch, sk, S, host27, dev, args.profile_steps)
        return 0

    head = run_headline(torch, sk, S, host27, args, stream, dev)
    del host27

    out = {
        "metric": METRIC,
        "value": round(head["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "layers": LAYERS, "m": [1, 8], "group": GROUP,
                   "weight_bytes_resident": int(head["weight_bytes"]),
                   "algorithmic_bytes_per_step": int(head["step_bytes"])},
        "frac_peak": round(head["value"] / PEAK_GBPS, 4),
        "m1": head["sweeps"][1],
        "m8": head["sweeps"][8],
        "m8_over_m1": round(head["sweeps"][8]["us_per_sweep"] / head["sweeps"][1]["us_per_sweep"], 4),
        "per_linear": head["per"],
        "layer_major": head["layer_major"],
        "instances": head["instances"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
    }
    if cpu_table is not None:
        out["cpu_oracle_configs"] = cpu_table

    if not args.no_9b:
        d9, host9, xs9, R9 = run_9b(torch, sk, S, dev, stream, args.copies,
                                    (1, 8) if args.no_sweep else tuple(range(1, 9)))
        out["decoder_9b"] = d9
        if not args.no_ablation:
            out["ablation"] = time_ablation(torch, sk, stream, host9, xs9, R9, d9["per_call"])
        del host9, xs9
    if not args.no_experts:
        out["experts"] = time_experts(torch, sk, S, stream)
    if not args.no_attention:
        out["attention"] = time_attention(torch, sk, S, stream)
    if not args.no_mtp:
        us1 = head["sweeps"][1]["us_per_sweep"]
        out["mtp"] = plan_mtp(sk, us1 / 1e3, head["sweeps"][8]["us_per_sweep"] / 1e3, us1 / LAYERS / 1e3)
    if not args.no_variants:
        out["variants"] = time_variants(torch, sk, S, dev, stream)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
