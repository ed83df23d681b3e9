#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s and µs/call of the W4A8 skinny GEMM on one MI355X.

Workload (one "step"): the four linears of a 9B-class decoder layer, W4A8 with
G = 32 and fp32 activations -- QKV 4096->6144, O 4096->4096, gate+up
4096->24576, down 12288->4096 -- first at M = 1 (plain decode), then at M = 8
(a verify pass with 7 draft rows).  Inputs are seeded synthetic tensors already
resident in HBM; weights are repacked once before timing.

Cold weights: MI355X has a 256 MB last-level cache, so every linear has R
repacked copies (same values, distinct addresses) and consecutive calls rotate
through them; more than 1 GiB of weights is touched between two reads of the
same copy.  Timing uses HIP graphs replayed on torch's current stream, with
HIP events recorded on that same stream.

Algorithmic bytes of one call: packed weights + FP32 scales + activations +
fp32 output.  Peak: 8 TB/s HBM3E.

Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s & µs/call, W4A8 skinny GEMM at M=1 and M=8 (frac. of peak)"
PEAK_GBPS = 8000.0
SHAPES = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096), ("down", 4096, 12288)]
GROUP = 32
CONFIG_ID = 1          # seed recipe: 1000*config + 10*linear + tensor id
COPY_PROBE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4_g32_decoder_layer_hbm_traffic.md")
# the sources the timed kernels are built from (kernel, launch planning, W4 instances),
# hashed in this order to tie the committed counter summary to them
KERNEL_SOURCES = ("sk_gemm_kernel.h", "sk_gemm.hip", "sk_gemm_w4.hip")


def measured_traffic(kernel_key: str):
    """HBM bytes per launch of `kernel_key` from the committed counter summary, or
    None when that summary was taken on a different kernel source."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "gemm_sk_repack_amd", "csrc", name), "rb").read())
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != h.hexdigest():
        return None
    m = re.search(r"traffic_bytes_per_launch\[" + re.escape(kernel_key) + r"\]:\s*([0-9]+)", text)
    return int(m.group(1)) if m else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(n: int, k: int, m: int, g: int = GROUP, xbytes: int = 4) -> int:
    return n * k // 2 + n * (k // g) * 4 + m * k * xbytes + m * n * 4


def time_graph(torch, stream, fn, calls):
    """µs per call of `calls` invocations of fn(i) captured in one HIP graph (median of 3).
    One eager call first: a call that grows the library's workspace must not be captured."""
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b) * 1e3 / calls)
    return float(np.median(t))


def time_experts(torch, sk, S, stream):
    """Expert-bank workload (synthetic): a W4A8 G=32 bank of 32 experts x 2048
    rows at K = 4096 (168 MB), 7 rotated copies (1.2 GB); M = 1 with 2 listed
    experts and M = 8 with 8, a fresh list per call.  One sk_gemm_experts
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
                    "GBps": round(b / (us_bank * 1e-6) / 1e9, 1),
                    "separate_launches_us": round(us_sep, 3),
                    "separate_GBps": round(b / (us_sep * 1e-6) / 1e9, 1)})
        log(f"experts M={m} x{nl}: one launch {us_bank:7.3f} us ({out[-1]['GBps']} GB/s), "
            f"{nl} launches {us_sep:7.3f} us")
    del views, banks, base
    return {"workload": ("synthetic W4A8 G=32 expert bank, 32 experts x 2048 rows, K = 4096, "
                         "7 rotated copies; a fresh expert list per call"),
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
            gbps = b / (us * 1e-6) / 1e9
            out.append({"L": length, "m": m, "us_per_call": round(us, 3),
                        "GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_GBPS, 4),
                        "ranges_per_head": splits, "blocks_per_range": bps})
            log(f"attention L={length} M={m}: {us:7.3f} us ({out[-1]['GBps']} GB/s), "
                f"{splits} ranges x {bps} blocks per head")
        del caches, base
    return {"workload": ("synthetic 9B-class GQA decode attention: Hq 32, Hkv 8, head dim 128, "
                         "bf16 KV cache (tiled), causal verification rows; rotated cache copies"),
            "per_call": out}


def plan_mtp(sk, t1_us: float, t8_us: float):
    """The library's tree-MTP planner on synthetic acceptance statistics, with
    this build's measured costs: verify = a 32-layer 9B-class forward at M = 8
    (32 x the decoder-layer linears step at M = 8), draft = one MTP layer at
    M = 1 (the linears step at M = 1).  Attention and the rest of the layer are
    left out on both sides.  Reports the layout the planner settles on, the mean
    tokens per step and the rate against plain decoding (32 layers at M = 1)."""
    rng = np.random.default_rng(0)
    regimes = {
        "code-like": [0.04, 0.86, 0.06, 0.02, 0.01, 0.005, 0.003, 0.002],
        "creative-like": [0.15, 0.35, 0.25, 0.13, 0.05, 0.03, 0.02, 0.02],
    }
    verify_ms, draft_ms = 32 * t8_us / 1e3, t1_us / 1e3
    plain_ms = 32 * t1_us / 1e3
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
    return {"verify_ms": round(verify_ms, 4), "draft_ms": round(draft_ms, 4),
            "note": ("synthetic rank statistics; costs from this run's decoder-layer linears "
                     "(32 layers at M = 8 to verify, one layer at M = 1 to draft)"),
            "regimes": out}


def time_ablation(torch, sk, stream, host, xs, R, per):
    """The same step on the split path: (a) the weight left in the canonical
    layout (codes and scales read from their two regions), quantising in the
    launch; (b) also quantising in a launch of its own, q and sx through
    memory.  µs per call from graphs over R rotated canonical copies."""
    dev = torch.device("cuda:0")
    rows = []
    tot = {"fused": 0.0, "canonical": 0.0, "split": 0.0}
    for name, n, k in SHAPES:
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
                         "fused_GBps": round(b / (us_fused * 1e-6) / 1e9, 1),
                         "split_GBps": round(b / (us_split * 1e-6) / 1e9, 1)})
            tot["fused"] += us_fused
            tot["canonical"] += us_can
            tot["split"] += us_split
            log(f"split path {name:8s} M={m}: fused {us_fused:7.3f}  canonical {us_can:7.3f}  "
                f"canonical + separate quantisation {us_split:7.3f} us/call")
        del cps, base
    return {"what": ("the step's 8 calls on (a) the weight in the canonical layout, quantising "
                     "in the launch, and (b) that plus quantisation as its own launch (q, sx "
                     "through memory), against the fused stream-layout path"),
            "step_us": {kk: round(v, 3) for kk, v in tot.items()},
            "speedup_of_fused": {"over_canonical": round(tot["canonical"] / tot["fused"], 4),
                                 "over_split": round(tot["split"] / tot["fused"], 4)},
            "per_call": rows}


def time_variants(torch, sk, S, dev, stream):
    """The other workloads: the single 1024 x 1024 linear, fused prologues at
    hidden 4096, the W6 / codebook / lm_head formats at K = 4096, and one
    27B-class layer (bf16 activations) whose 64-layer step time is extrapolated
    from that layer."""
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
                     "us_per_call": round(us, 3), "GBps": round(alg / (us * 1e-6) / 1e9, 1),
                     "frac_peak": round(alg / (us * 1e-6) / 1e9 / PEAK_GBPS, 4)})
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

    # fused prologues at hidden 4096
    cps, nb = weight_copies(sk.SK_W4_SYM, 6144, 4096, 32, 3, 0)
    gam = torch.from_numpy(S.gamma(S.seed_of(3, 0, S.TENSOR_GAMMA), 4096)).to(dev)
    for m in (1, 3, 8):
        x = torch.from_numpy(S.activations(S.seed_of(3, 0, S.TENSOR_X), m, 4096)).to(dev)
        y = torch.empty((m, 6144), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_fused_rmsnorm(
            cps[i % len(cps)], x, gam, 1e-6, y=y), 4 * len(cps))
        record("fused", "rmsnorm+qkv", 6144, 4096, 32, 0, m, us, nb, extra=4096 * 4)
    cps, nb = weight_copies(sk.SK_W4_SYM, 4096, 12288, 32, 3, 1)
    for m in (1, 3, 8):
        gu = torch.from_numpy(np.concatenate(
            [S.activations(S.seed_of(3, 1, S.TENSOR_GATE), m, 12288),
             S.activations(S.seed_of(3, 1, S.TENSOR_UP), m, 12288)], axis=1)).to(dev)
        y = torch.empty((m, 4096), dtype=torch.float32, device=dev)
        us = time_graph(torch, stream, lambda i: sk.sk_gemm_fused_swiglu(
            cps[i % len(cps)], gu[:, :12288], gu[:, 12288:], y=y), 4 * len(cps))
        record("fused", "swiglu+down", 4096, 12288, 32, 0, m, us, nb, extra=m * 12288 * 4,
               xbytes=4)
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
            us = time_graph(torch, stream, lambda i: fn(cps[i % len(cps)], x, y=y),
                            max(8, 2 * len(cps)))
            record("formats", name, n, 4096, g, fmt, m, us, nb)
        del cps
    # one 27B-class layer, bf16 activations; the 64-layer step is 64 x the layer
    layer = [("qkv", 7168, 5120), ("o", 5120, 5120), ("gate_up", 34816, 5120),
             ("down", 5120, 17408)]
    for m in (1, 8):
        tot_us = tot_b = 0.0
        for li, (name, n, k) in enumerate(layer):
            cps, nb = weight_copies(sk.SK_W4_SYM, n, k, 32, 2, li)
            bits = S.to_bf16_bits(S.activations(S.seed_of(2, li, S.TENSOR_X), m, k))
            x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            us = time_graph(torch, stream, lambda i: sk.sk_gemm_w4a8(cps[i % len(cps)], x, y=y),
                            4 * len(cps))
            record("27b_layer", name, n, k, 32, 0, m, us, nb, xbytes=2)
            tot_us += us
            tot_b += nb + m * k * 2 + m * n * 4
            del cps
        rows.append({"group": "27b_step_extrapolated", "m": m, "layers": 64,
                     "us_per_step": round(64 * tot_us, 1),
                     "GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
                     "note": "64 x the measured layer (lm_head excluded)"})
    return rows


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=10, help="rotated weight copies per linear")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the per-shape M sweep")
    ap.add_argument("--profile-calls", type=int, default=0,
                    help="run this many eager steps (no graphs, no timing) and exit: the "
                         "workload for rocprofv3 kernel traces and counters")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other workloads (fused prologues, W6 / codebook / lm_head "
                         "formats, the 27B-class layer) reported as `variants`")
    ap.add_argument("--no-experts", action="store_true",
                    help="skip the expert-bank workload")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the decode-attention workload")
    ap.add_argument("--no-mtp", action="store_true",
                    help="skip the tree-MTP planning summary")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the split-path comparison (canonical layout, separate quantisation)")
    ap.add_argument("--profile-attention", type=int, default=0,
                    help="run this many eager decode-attention calls (L = 16384, M = 1 and 8, "
                         "rotated caches) and exit: the workload for its rocprofv3 kernel trace")
    ap.add_argument("--copy-probe", action="store_true",
                    help="copy a 256 MiB device buffer 5 times and exit: the known-size "
                         "kernel that calibrates the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures the skinny GEMM on one GPU; --gpus above 1 is not supported "
              "(the workload runs on a single MI355X)", file=sys.stderr)
        return 2

    import torch

    import gemm_sk_repack_amd as sk
    import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
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
    R = args.copies
    if R % 2:
        R += 1

    # ---------------- inputs ----------------
    t0 = time.time()
    host = {}
    weights = {}
    for li, (name, n, k) in enumerate(SHAPES):
        _, _, buf = S.make_weight(S.FMT_W4, n, k, GROUP, S.seed_of(CONFIG_ID, li, S.TENSOR_W),
                                  S.seed_of(CONFIG_ID, li, S.TENSOR_S))
        host[name] = buf
        base = sk.QuantWeight(torch.from_numpy(buf).to(dev), n, k, GROUP, sk.SK_W4_SYM)
        sk.sk_repack_w4a8(base)
        copies = [base]
        for _ in range(R - 1):
            c = sk.QuantWeight(base.data.clone(), n, k, GROUP, sk.SK_W4_SYM)
            c.desc.layout = sk.SK_LAYOUT_STREAM          # bytes cloned from a repacked weight
            copies.append(c)
        weights[name] = copies
    xs = {}
    for m in range(1, 9):
        for k in sorted({k for _, _, k in SHAPES}):
            xs[(m, k)] = torch.from_numpy(S.activations(S.seed_of(CONFIG_ID, m, S.TENSOR_X) + k, m, k)).to(dev)
    ys = {(name, m): torch.empty((m, n), dtype=torch.float32, device=dev)
          for name, n, _ in SHAPES for m in range(1, 9)}
    torch.cuda.synchronize()
    wbytes = sum(w.data.numel() for c in weights.values() for w in c)
    log(f"setup {time.time() - t0:.1f}s, {R} copies per linear, {wbytes / 2**30:.2f} GiB of weights")

    def call(name, m, copy):
        _, n, k = next(s for s in SHAPES if s[0] == name)
        sk.sk_gemm_w4a8(weights[name][copy % R], xs[(m, k)], y=ys[(name, m)])

    def step(s):
        for name, _, _ in SHAPES:
            call(name, 1, 2 * s)
        for name, _, _ in SHAPES:
            call(name, 8, 2 * s + 1)

    step_bytes = sum(alg_bytes(n, k, m) for _, n, k in SHAPES for m in (1, 8))

    if args.profile_calls:
        for s in range(args.profile_calls):
            step(s)
        torch.cuda.synchronize()
        log(f"profile run: {args.profile_calls} eager steps of {2 * len(SHAPES)} calls")
        return 0

    # ---------------- warmup (eager), then capture the timed steps ----------------
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(args.steps):
            step(args.warmup + s)
    graph.replay()                 # one untimed replay: first-replay costs stay outside
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = e0.elapsed_time(e1)
    ms_per_step = elapsed_ms / args.steps
    value = step_bytes * args.steps / (elapsed_ms * 1e-3) / 1e9
    log(f"timed {args.steps} steps: {elapsed_ms:.3f} ms, {ms_per_step * 1e3:.2f} us/step, {value:.0f} GB/s")

    # ---------------- per (linear, M) µs/call ----------------
    spread = {}                    # (linear, M) -> (p10, p90) of the 7 replays

    def time_calls(name, m, reps=4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps * R):
                call(name, m, r)
        g.replay()
        torch.cuda.synchronize()
        best = []
        for _ in range(7):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            best.append(a.elapsed_time(b) * 1e3 / (reps * R))
        spread[(name, m)] = (float(np.percentile(best, 10)), float(np.percentile(best, 90)))
        return float(np.median(best))

    # the streaming-read probe on the same rotated weight buffers: the best of a
    # few launch shapes, as the ceiling a kernel reading those bytes can reach
    probe_out = torch.zeros(4, dtype=torch.int32, device=dev)

    def time_probe(name, reps=4):
        best_us = None
        for grid in (256, 512, 1024, 2048):
            for threads in (256, 1024):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for r in range(reps * R):
                        sk.stream_read(weights[name][r % R].data, grid, threads, probe_out)
                g.replay()
                torch.cuda.synchronize()
                t = []
                for _ in range(3):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    g.replay()
                    b.record(stream)
                    torch.cuda.synchronize()
                    t.append(a.elapsed_time(b) * 1e3 / (reps * R))
                us = float(np.median(t))
                best_us = us if best_us is None else min(best_us, us)
        return best_us

    probe = {}
    for name, n, k in SHAPES:
        probe[name] = time_probe(name)
        nb = weights[name][0].data.numel()
        log(f"probe    {name:8s}: {probe[name]:8.3f} us to read its {nb / 1e6:.1f} MB of weights "
            f"({nb / (probe[name] * 1e-6) / 1e9:.0f} GB/s)")

    ms_list = (1, 8) if args.no_sweep else tuple(range(1, 9))
    per = []
    for name, n, k in SHAPES:
        for m in ms_list:
            us = time_calls(name, m)
            b = alg_bytes(n, k, m)
            per.append({"linear": name, "n": n, "k": k, "m": m, "us_per_call": round(us, 3),
                        "us_p10": round(spread[(name, m)][0], 3), "us_p90": round(spread[(name, m)][1], 3),
                        "GBps": round(b / (us * 1e-6) / 1e9, 1),
                        "frac_peak": round(b / (us * 1e-6) / 1e9 / PEAK_GBPS, 4),
                        "probe_us": round(probe[name], 3),
                        "frac_of_probe": round(probe[name] / us, 4)})
            log(f"{name:8s} M={m}: {us:8.3f} us/call  {per[-1]['GBps']:7.1f} GB/s  "
                f"({100 * per[-1]['frac_peak']:.1f}% of peak, {100 * per[-1]['frac_of_probe']:.0f}% of the probe)")

    def agg(m):
        rows = [p for p in per if p["m"] == m]
        us = sum(p["us_per_call"] for p in rows)
        b = sum(alg_bytes(p["n"], p["k"], m) for p in rows)
        return us, b

    us1, b1 = agg(1)
    us8, b8 = agg(8)
    # the dominant kernel: the template instance with the larger share of the step
    dom_m = 1 if us1 >= us8 else 8
    dom_us, dom_b = (us1, b1) if dom_m == 1 else (us8, b8)
    achieved = dom_b / (dom_us * 1e-6) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4), "traffic": measured_traffic(f"m{dom_m}"),
        "kernel": ("gemm_kernel<W4, no prologue, f32, G32, dot4, no exports> (all M=1 calls)" if dom_m == 1
                   else "gemm_kernel<W4, no prologue, f32, G32, MFMA, no exports> (all M=8 calls)"),
        "bytes_per_launch": dom_b // len(SHAPES),
        "us_per_launch": round(dom_us / len(SHAPES), 3),
    }

    # ---------------- split path: what the stream layout and fusion buy ----------------
    ablation = None
    if not args.no_ablation:
        ablation = time_ablation(torch, sk, stream, host, xs, R, per)

    experts = None
    if not args.no_experts:
        experts = time_experts(torch, sk, S, stream)

    attention = None
    if not args.no_attention:
        attention = time_attention(torch, sk, S, stream)

    mtp = None
    if not args.no_mtp:
        mtp = plan_mtp(sk, us1, us8)

    # ---------------- CPU baseline: the oracle on one step ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        xs_host = {key: v.cpu().numpy() for key, v in xs.items()}
        # whole steps (the 4 linears at M=1 and at M=8) until about 10 s of CPU work
        t_start = time.perf_counter()
        nsteps = 0
        while nsteps < 10 and (nsteps == 0 or time.perf_counter() - t_start < 10.0):
            for m in (1, 8):
                for name, n, k in SHAPES:
                    O.reference(0, host[name], n, k, GROUP, xs_host[(m, k)])
            nsteps += 1
        cpu_s = time.perf_counter() - t_start
        cpu = {"value": round(nsteps * step_bytes / cpu_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": (f"{nsteps} full steps (the 4 linears at M=1 and at M=8) through the numpy "
                          f"oracle, {cpu_s:.1f} s single-threaded on {platform.processor() or 'host'} "
                          f"({len(os.sched_getaffinity(0))} cores visible)")}
        log(f"cpu oracle: {cpu_s:.1f}s for {nsteps} steps -> {cpu['value']} GB/s")

    variants = None if args.no_variants else time_variants(torch, sk, S, dev, stream)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": ("9B-class decoder layer linears, W4A8 G=32, fp32 activations: QKV 4096->6144, "
                         "O 4096->4096, gate+up 4096->24576, down 12288->4096; one step = the 4 "
                         "linears at M=1 then at M=8"),
            "global_batch": 1, "weight_copies_rotated": R,
            "weight_bytes_resident": int(wbytes),
        },
        "frac_peak": round(value / PEAK_GBPS, 4),
        "m1": {"us_per_layer": round(us1, 3), "GBps": round(b1 / (us1 * 1e-6) / 1e9, 1)},
        "m8": {"us_per_layer": round(us8, 3), "GBps": round(b8 / (us8 * 1e-6) / 1e9, 1)},
        "m8_over_m1": round(us8 / us1, 4),
        "per_call": per,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if ablation is not None:
        out["ablation"] = ablation
    if experts is not None:
        out["experts"] = experts
    if attention is not None:
        out["attention"] = attention
    if mtp is not None:
        out["mtp"] = mtp
    if variants is not None:
        out["variants"] = variants
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
