#!/usr/bin/env python3
"""Benchmark: HSTU jagged causal attention forward on one MI355X.

One step = one hstu_attn_fwd call (work-list kernel + attention kernel) over
the whole batch, inputs resident in HBM.  Default workload: 16 sequences of
4096 tokens, heads 4, d 64, bf16 (the QKV (16, 4, 4096, 64) shape the Ascend
HSTU blog times in §2.2, §3.2 and §5.2), re-laid as a jagged batch.

Prints one JSON line.  `value` is useful TFLOP/s: 4 * heads * d *
sum_i s_i (s_i + 1) / 2 per call over the measured call time.  The roofline
object reports the attention kernel's own average duration (HIP events the
library records on the call's stream during the timed region).  The
cpu_baseline object times the fp64 CPU oracle on a bounded sample of the same
workload.

--targets times hstu_attn_fwd_targets instead, on 16 users x (3072 history +
1024 candidates) (the target-aware mask of M-FALCON ranking, HSTU paper
translation Appendix H); useful FLOPs then count the pairs that mask keeps.  --cached times
hstu_attn_fwd_cached on 16 users x (3072 cached history rows, 1024 candidates)
(M-FALCON's later micro-batches): t (h + 1) pairs per request.  --backward
times hstu_attn_bwd (dq, dk, dv) on the 16 x 4096 workload: useful FLOPs are
the five products of a recomputing backward, 10 * heads * d per kept pair
(2.5x the forward's); the kernels run seven (S and dP are formed by both the
dK/dV and the dQ kernel).  --rab times hstu_attn_fwd_rab (the relative
attention bias, HSTU paper translation §3 and Appendix G) on the 16 x 4096
workload with a position entry per distance and 16 time buckets; useful FLOPs
are the plain forward's (the bias terms are not counted); --backward --rab
times hstu_attn_bwd_rab (dq, dk, dv and both tables' gradients) on it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
PEAK_HBM_GBS = 8000.0
METRIC = "HSTU attn fwd useful TFLOP/s, % bf16 MFMA peak; ms at QKV(16,4,4096,64)"
METRIC_TARGETS = "HSTU target-aware attn fwd useful TFLOP/s (M-FALCON mask)"
METRIC_DENSE = "HSTU attn fwd useful TFLOP/s, dense (b, heads, s, d) layout"
METRIC_BWD = "HSTU attn bwd (dq, dk, dv) useful TFLOP/s"
METRIC_CACHED = "HSTU cached-history attn fwd useful TFLOP/s (M-FALCON micro-batch)"
METRIC_RAB = "HSTU attn fwd with relative attention bias useful TFLOP/s"
METRIC_RAB_TARGETS = ("HSTU target-aware attn fwd with relative attention bias useful TFLOP/s "
                      "(M-FALCON mask and bias)")
METRIC_RAB_CACHED = ("HSTU cached-history attn fwd with relative attention bias useful TFLOP/s "
                     "(M-FALCON micro-batch)")
METRIC_RAB_BWD = "HSTU attn bwd with relative attention bias (dq, dk, dv, table gradients) useful TFLOP/s"
# HBM traffic per dispatch of the attention kernel, from two rocprofv3 --pmc
# runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# same counter reads for a plain 1 GiB device copy (bench.py --copy-calibrate):
# FETCH_SIZE reads 0.5 GiB for that copy's 1 GiB of reads, WRITE_SIZE 1 GiB.
# The figures hold for the kernel and work-list sources with the SHA-256 below
# (the queue order decides which key/value re-reads hit the L2); for any other
# sources the bench reports traffic as null.
TRAFFIC = {
    "sources": ("generative_recommendation_attention_amd/csrc/attn_fwd.hip",
                "generative_recommendation_attention_amd/csrc/schedule.h",
                "generative_recommendation_attention_amd/csrc/schedule.hip"),
    "sha256": "ee703a20371daf55b3106a940942e2629fd849947452290a65960569e7976662",
    "fetch_scale": 2.0,
    "write_scale": 1.0,
    # mean over the launches that take the timed calls' form
    "fetch_kib": {1: 294.0, 2: 94499.5, 3: 1234048.4, 4: 387225.0, 5: 397324.7},
    "write_kib": {1: 200.7, 2: 39525.2, 3: 141251.6, 4: 54574.7, 5: 264980.7},
}


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(workload: int):
    if sources_sha256() != TRAFFIC["sha256"] or workload not in TRAFFIC["fetch_kib"]:
        return None
    kib = (TRAFFIC["fetch_kib"][workload] * TRAFFIC["fetch_scale"] +
           TRAFFIC["write_kib"][workload] * TRAFFIC["write_scale"])
    return round(kib * 1024.0)


def to_device(case):
    import torch
    def conv(x):
        if case.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return (conv(case.q), conv(case.k), conv(case.v),
            torch.from_numpy(case.offsets.astype(np.int32)).cuda())


def seen_pairs(case) -> float:
    """(query, key) pairs the mask keeps, summed over sequences: s(s+1)/2 for
    the causal mask; with t candidates after a history of h = s - t tokens,
    h(h+1)/2 for the history rows plus h + 1 for each candidate."""
    s = case.lengths.astype(np.float64)
    if case.num_targets is None:
        return float(np.sum(s * (s + 1.0) / 2.0))
    t = np.clip(case.num_targets.astype(np.float64), 0.0, s)
    h = s - t
    return float(np.sum(h * (h + 1.0) / 2.0 + t * (h + 1.0)))


def cpu_baseline_cached(cc, budget_s: float, rab=None, hist_ts=None):
    """The oracle's cached-history form (with the relative attention bias when
    rab is given) on whole requests, in input order, until about budget_s of
    wall time has been spent."""
    import oracle
    lib = oracle.load()
    threads = oracle.threads(lib)
    c = cc.cand
    per_call = max(1, -(-threads // c.heads))
    done_flops, done_s, seqs, i = 0.0, 0.0, 0, 0
    while i < c.num_seqs and done_s < budget_s:
        j = min(c.num_seqs, i + per_call)
        a, b = int(c.offsets[i]), int(c.offsets[j])
        ha, hb = int(cc.hist_offsets[i]), int(cc.hist_offsets[j])
        t0 = time.perf_counter()
        if rab is None:
            oracle.fwd_cached(c.q[a:b], c.k[a:b], c.v[a:b], c.offsets[i:j + 1] - c.offsets[i],
                              cc.k_cache[ha:hb], cc.v_cache[ha:hb],
                              cc.hist_offsets[i:j + 1] - cc.hist_offsets[i], c.heads, c.d,
                              c.alpha, c.n, c.dtype, lib=lib)
        else:
            oracle.fwd_rab_cached(c.q[a:b], c.k[a:b], c.v[a:b], c.offsets[i:j + 1] - c.offsets[i],
                                  cc.k_cache[ha:hb], cc.v_cache[ha:hb],
                                  cc.hist_offsets[i:j + 1] - cc.hist_offsets[i],
                                  rab.timestamps[a:b], hist_ts[ha:hb], rab.pos_bias,
                                  rab.time_bias, c.heads, c.d, c.alpha, c.n, c.dtype, lib=lib)
        done_s += time.perf_counter() - t0
        t = c.lengths[i:j].astype(np.float64)
        h = cc.hist_lengths[i:j].astype(np.float64)
        done_flops += float(np.sum(4.0 * c.heads * c.d * t * (h + 1.0)))
        seqs += j - i
        i = j
    return {"value": done_flops / done_s / 1e12, "unit": "TFLOP/s",
            "cores": min(threads, per_call * c.heads), "kind": "oracle",
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{seqs} of {c.num_seqs} requests, all heads; fp64 loop oracle "
                      f"(OpenMP over (request, head)), {done_s:.1f} s wall, "
                      f"{threads} threads available"}


def cpu_baseline_bwd(case, dout, budget_s: float, rab=None):
    """The oracle's backward on whole sequences, in input order, until about
    budget_s of wall time has been spent."""
    import oracle
    lib = oracle.load()
    threads = oracle.threads(lib)
    off = case.offsets
    per_call = max(1, -(-threads // case.heads))
    done_flops, done_s, seqs, i = 0.0, 0.0, 0, 0
    while i < case.num_seqs and done_s < budget_s:
        j = min(case.num_seqs, i + per_call)
        a, b = int(off[i]), int(off[j])
        tg = None if case.num_targets is None else case.num_targets[i:j]
        t0 = time.perf_counter()
        if rab is not None:
            oracle.bwd_rab(case.q[a:b], case.k[a:b], case.v[a:b], dout[a:b],
                           off[i:j + 1] - off[i], rab.timestamps[a:b], rab.pos_bias,
                           rab.time_bias, case.heads, case.d, case.alpha, case.n, case.dtype,
                           lib=lib, num_targets=tg)
        else:
            oracle.bwd(case.q[a:b], case.k[a:b], case.v[a:b], dout[a:b], off[i:j + 1] - off[i],
                       case.heads, case.d, case.alpha, case.n, case.dtype, lib=lib,
                       num_targets=tg)
        done_s += time.perf_counter() - t0
        part = workloads.Case(name="", dtype=case.dtype, heads=case.heads, d=case.d,
                              offsets=off[i:j + 1] - off[i], q=case.q[:0], k=case.k[:0],
                              v=case.v[:0], alpha=case.alpha, n=case.n, num_targets=tg)
        done_flops += 10.0 * case.heads * case.d * seen_pairs(part)
        seqs += j - i
        i = j
    return {"value": done_flops / done_s / 1e12, "unit": "TFLOP/s",
            "cores": min(threads, per_call * case.heads), "kind": "oracle",
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{seqs} of {case.num_seqs} sequences, all heads; fp64 loop oracle "
                      f"backward (OpenMP over (sequence, head)), {done_s:.1f} s wall, "
                      f"{threads} threads available"}


def cpu_baseline(case, budget_s: float, rab=None):
    """Time the oracle on whole sequences of the workload (all heads).  Each
    oracle call takes enough sequences to give every OpenMP thread a
    (sequence, head) pair; calls continue in input order until about budget_s
    of wall time has been spent."""
    import oracle
    lib = oracle.load()
    threads = oracle.threads(lib)
    off = case.offsets
    per_call = max(1, -(-threads // case.heads))
    done_flops, done_s, seqs = 0.0, 0.0, 0
    i = 0
    while i < case.num_seqs and done_s < budget_s:
        j = min(case.num_seqs, i + per_call)
        a, b = int(off[i]), int(off[j])
        sub = (off[i:j + 1] - off[i]).astype(np.int32)
        t0 = time.perf_counter()
        tg = None if case.num_targets is None else case.num_targets[i:j]
        if rab is not None:
            oracle.fwd_rab(case.q[a:b], case.k[a:b], case.v[a:b], sub, rab.timestamps[a:b],
                           rab.pos_bias, rab.time_bias, case.heads, case.d, case.alpha, case.n,
                           case.dtype, lib=lib, num_targets=tg)
        else:
            oracle.fwd(case.q[a:b], case.k[a:b], case.v[a:b], sub, case.heads, case.d,
                       case.alpha, case.n, case.dtype, lib=lib, num_targets=tg)
        done_s += time.perf_counter() - t0
        part = workloads.Case(name="", dtype=case.dtype, heads=case.heads, d=case.d,
                              offsets=sub, q=case.q[:0], k=case.k[:0], v=case.v[:0],
                              alpha=case.alpha, n=case.n, num_targets=tg)
        done_flops += 4.0 * case.heads * case.d * seen_pairs(part)
        seqs += j - i
        i = j
    used = min(threads, per_call * case.heads)
    return {"value": done_flops / done_s / 1e12, "unit": "TFLOP/s", "cores": used,
            "kind": "oracle", "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{seqs} of {case.num_seqs} sequences, all heads; fp64 loop oracle "
                      f"(OpenMP over (sequence, head)), {done_s:.1f} s wall, "
                      f"{threads} threads available"}


def bench_layer(args) -> int:
    """One layer forward: hstu_layer_in_proj, hstu_attn_fwd, hstu_layer_out_proj
    on the chosen workload with d_model = heads * d (bf16/fp16).  Reports the
    whole layer's time and each part's own (each part timed alone, same
    inputs), with the projections' HBM rates."""
    import torch
    import generative_recommendation_attention_amd as hstu
    torch.cuda.set_device(0)
    case = workloads.workload(args.workload)
    if case.dtype == "fp32":
        print("--layer needs a bf16 or fp16 workload", file=sys.stderr)
        return 2
    T, H, D = case.total, case.heads, case.d
    hd = H * D
    dm = hd
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float16
    g = torch.Generator(device="cuda").manual_seed(3000)
    x = torch.randn((T, dm), generator=g, device="cuda").to(tdt)
    w1 = (torch.randn((4 * hd, dm), generator=g, device="cuda") / dm ** 0.5).to(tdt)
    b1 = 0.1 * torch.randn(4 * hd, generator=g, device="cuda")
    w2 = (torch.randn((dm, hd), generator=g, device="cuda") / hd ** 0.5).to(tdt)
    gamma = 1.0 + 0.1 * torch.randn(hd, generator=g, device="cuda")
    beta = 0.1 * torch.randn(hd, generator=g, device="cuda")
    b2 = 0.1 * torch.randn(dm, generator=g, device="cuda")
    off = torch.from_numpy(case.offsets.astype(np.int32)).cuda()
    uvqk = tuple(torch.empty((T, H, D), dtype=tdt, device="cuda") for _ in range(4))
    attn = torch.empty((T, H, D), dtype=tdt, device="cuda")
    y = torch.empty_like(x)

    def p_in():
        hstu.hstu_layer_in_proj(x, w1, b1, H, D, out=uvqk)

    def p_attn():
        hstu.hstu_attn_fwd(uvqk[2], uvqk[3], uvqk[1], off, case.alpha, case.n, out=attn)

    def p_out():
        hstu.hstu_layer_out_proj(attn, uvqk[0], x, gamma, beta, 1e-5, w2, b2, out=y)

    def layer():
        p_in()
        p_attn()
        p_out()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_layer = timed(layer)
    ms_in, ms_attn, ms_out = timed(p_in), timed(p_attn), timed(p_out)
    elt = 2
    flops_attn = case.useful_flops()
    flops_in = 2.0 * T * dm * 4 * hd
    flops_out = 2.0 * T * hd * dm
    bytes_in = elt * (T * dm + 4 * hd * dm + 4 * T * hd) + 4 * 4 * hd
    bytes_out = elt * (2 * T * hd + 2 * T * dm + dm * hd) + 4 * (2 * hd + dm)
    total = flops_attn + flops_in + flops_out
    line = {
        "metric": "HSTU layer fwd (projections + attention) useful TFLOP/s",
        "value": round(total / (ms_layer * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_layer, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": case.description, "d_model": dm, "heads": H, "d": D,
                   "total_tokens": T},
        "parts": {
            "in_proj": {"ms": round(ms_in, 5), "hbm_GBps": round(bytes_in / ms_in / 1e6, 1),
                        "hbm_frac": round(bytes_in / ms_in / 1e6 / PEAK_HBM_GBS, 4),
                        "tflops": round(flops_in / ms_in / 1e9, 1)},
            "attention": {"ms": round(ms_attn, 5),
                          "tflops": round(flops_attn / ms_attn / 1e9, 1)},
            "out_proj": {"ms": round(ms_out, 5), "hbm_GBps": round(bytes_out / ms_out / 1e6, 1),
                         "hbm_frac": round(bytes_out / ms_out / 1e6 / PEAK_HBM_GBS, 4),
                         "tflops": round(flops_out / ms_out / 1e9, 1)},
        },
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    # From idle, the chip's power management takes some 50-100 ms of
    # back-to-back calls to reach its steady state (the forward on 16 x 4096
    # runs 0.24 ms per call over the first 25 calls, 0.19 ms after 400): before
    # the warm-up steps, calls are made until this much wall time has passed.
    # Reported as clock_settle in the JSON line; 0 turns it off.
    ap.add_argument("--settle-s", type=float, default=0.25)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--targets", action="store_true",
                    help="time the target-aware forward on 16 x (3072 history + 1024 candidates)")
    ap.add_argument("--layer", action="store_true",
                    help="time one HSTU layer forward (input projection, attention, output "
                         "projection) on the 16 x 4096 workload with d_model = heads * d")
    ap.add_argument("--dense", action="store_true",
                    help="time hstu_attn_fwd_dense on the chosen workload's shape laid out "
                         "(batch, heads, seq_len, d) (equal lengths only)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (dq, dk, dv) on the chosen workload")
    ap.add_argument("--cached", action="store_true",
                    help="time the cached-history forward on 16 x (3072 cached rows, "
                         "1024 candidates)")
    ap.add_argument("--rab", action="store_true",
                    help="time the forward with the relative attention bias on 16 x 4096 "
                         "(a position entry per distance, 16 time buckets); with --targets, "
                         "the target-aware forward with the bias on the --targets workload; "
                         "with --backward, the backward with the bias")
    ap.add_argument("--graph", action="store_true",
                    help="record one call into a HIP graph (torch.cuda.CUDAGraph) and time its "
                         "replays instead of eager calls (the library's kernel timers are off "
                         "under capture, so the roofline uses the whole replay)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="run only a plain 1 GiB device copy (3 times), the reference for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    modes = args.targets + args.cached + args.backward + args.dense + args.layer + args.rab
    if modes > 1 and (args.dense or args.layer or
                      (args.cached and modes - args.rab > 1)):
        ap.error("--dense and --layer are separate benchmarks; --cached combines with --rab "
                 "only; --targets, --backward and --rab combine")
    if args.graph and args.layer:
        ap.error("--graph records the attention calls; --layer has no graph form here")
    if args.layer:
        return bench_layer(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would run its own share of sequences with no exchange).",
              file=sys.stderr)
        return 2

    import torch
    import generative_recommendation_attention_amd as hstu

    torch.cuda.set_device(0)
    if args.copy_calibrate:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "copies": 3}), flush=True)
        return 0
    cc = rab = hist_ts = None
    if args.cached and args.rab:
        cc, rab, hist_ts = workloads.rab_cached_workload()
        case = cc.cand
    elif args.cached:
        cc = workloads.cached_workload()
        case = cc.cand
    elif args.rab and args.targets:
        case, rab = workloads.rab_targets_workload()
    elif args.rab:
        case, rab = workloads.rab_workload()
    elif args.targets:
        case = workloads.targets_workload()
    else:
        case = workloads.workload(args.workload)
    q, k, v, off = to_device(case)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    flops = 4.0 * case.heads * case.d * seen_pairs(case)
    alg_bytes = case.algorithmic_bytes()
    if args.cached:
        hist_case = workloads.Case(name="", dtype=case.dtype, heads=case.heads, d=case.d,
                                   offsets=cc.hist_offsets, q=cc.k_cache, k=cc.k_cache,
                                   v=cc.v_cache, alpha=case.alpha, n=case.n)
        kc, vc, hoff = to_device(hist_case)[1:]
        t = case.lengths.astype(np.float64)
        flops = float(np.sum(4.0 * case.heads * case.d * t * (cc.hist_lengths + 1.0)))
        elt = 4 if case.dtype == "fp32" else 2
        alg_bytes += 2.0 * elt * cc.k_cache.size + 4 * (case.num_seqs + 1)
        if args.rab:
            ts = torch.from_numpy(rab.timestamps).cuda()
            hts = torch.from_numpy(hist_ts).cuda()
            wp = torch.from_numpy(rab.pos_bias).cuda()
            wt = torch.from_numpy(rab.time_bias).cuda()
            alg_bytes += 4.0 * (case.total + hist_ts.size) + 4.0 * (rab.pos_bias.size +
                                                                     rab.time_bias.size)

            def call():
                hstu.hstu_attn_fwd_rab_cached(q, k, v, off, kc, vc, hoff, ts, hts, wp, wt,
                                              case.alpha, case.n, out=out)
        else:
            def call():
                hstu.hstu_attn_fwd_cached(q, k, v, off, kc, vc, hoff, case.alpha, case.n,
                                          out=out)
    elif args.rab and not args.backward:
        ts = torch.from_numpy(rab.timestamps).cuda()
        wp = torch.from_numpy(rab.pos_bias).cuda()
        wt = torch.from_numpy(rab.time_bias).cuda()
        alg_bytes += 4.0 * case.total + 4.0 * (rab.pos_bias.size + rab.time_bias.size)
        if args.targets:
            tg = torch.from_numpy(case.num_targets.astype(np.int32)).cuda()
            alg_bytes += 4.0 * case.num_seqs

            def call():
                hstu.hstu_attn_fwd_rab_targets(q, k, v, off, tg, ts, wp, wt, case.alpha, case.n,
                                               out=out)
        else:
            def call():
                hstu.hstu_attn_fwd_rab(q, k, v, off, ts, wp, wt, case.alpha, case.n, out=out)
    elif args.targets and not args.backward:
        tg = torch.from_numpy(case.num_targets.astype(np.int32)).cuda()

        def call():
            hstu.hstu_attn_fwd_targets(q, k, v, off, tg, case.alpha, case.n, out=out)
    elif args.dense:
        L = case.lengths
        if L.size == 0 or np.any(L != L[0]):
            ap.error("--dense needs a workload of equal lengths")
        B, S, H, D = case.num_seqs, int(L[0]), case.heads, case.d
        qd, kd, vd = (x.reshape(B, S, H, D).permute(0, 2, 1, 3).contiguous()
                      for x in (q, k, v))
        outd = torch.empty_like(qd)

        def call():
            hstu.hstu_attn_fwd_dense(qd, kd, vd, case.alpha, case.n, out=outd)
    elif args.backward:
        dout_host = workloads.make_case(list(case.lengths), case.heads, case.d, case.dtype,
                                        seed=2000).q
        dout = to_device(workloads.Case(name="", dtype=case.dtype, heads=case.heads, d=case.d,
                                        offsets=case.offsets, q=dout_host, k=dout_host,
                                        v=dout_host, alpha=case.alpha, n=case.n))[0]
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
        flops *= 2.5
        # q, k, v, dout read once, dq, dk, dv written once
        alg_bytes *= 7.0 / 4.0
        tg = None
        if args.targets:
            tg = torch.from_numpy(case.num_targets.astype(np.int32)).cuda()
            alg_bytes += 4.0 * case.num_seqs
        if args.rab:
            ts = torch.from_numpy(rab.timestamps).cuda()
            wp = torch.from_numpy(rab.pos_bias).cuda()
            wt = torch.from_numpy(rab.time_bias).cuda()
            rgrads = grads + (torch.empty_like(wp), torch.empty_like(wt))
            alg_bytes += 4.0 * case.total + 8.0 * (rab.pos_bias.size + rab.time_bias.size)
            if tg is not None:
                def call():
                    hstu.hstu_attn_bwd_rab_targets(q, k, v, dout, off, tg, ts, wp, wt,
                                                   case.alpha, case.n, grads=rgrads)
            else:
                def call():
                    hstu.hstu_attn_bwd_rab(q, k, v, dout, off, ts, wp, wt, case.alpha, case.n,
                                           grads=rgrads)
        else:
            def call():
                hstu.hstu_attn_bwd(q, k, v, dout, off, case.alpha, case.n, grads=grads,
                                   num_targets=tg)
    else:
        def call():
            hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n, out=out)

    settle_calls = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            call()
        settle_calls += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    if args.graph:
        eager_call = call
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            eager_call()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_call()
        torch.cuda.synchronize()

        def call():
            graph.replay()
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()

    hstu.hstu_profile_read(reset=True)
    hstu.hstu_profile_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    hstu.hstu_profile_enable(False)
    total_ms = start.elapsed_time(end)
    kt = hstu.hstu_profile_read(reset=True)
    ms = total_ms / args.steps
    value = flops / (ms * 1e-3) / 1e12

    attn_ms = kt.attn_ms / max(1, kt.calls) if kt.calls else ms
    sched_ms = kt.sched_ms / max(1, kt.calls)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[case.dtype]
    traffic = (None if (args.targets or args.cached or args.backward or args.dense or args.rab or
                        args.graph) else traffic_bytes(args.workload))
    # The bound is the roofline the workload's arithmetic intensity (useful
    # FLOPs per algorithmic byte) falls under: HBM below the ridge point
    # (peak FLOP/s over 8 TB/s), the matrix cores above it.
    hbm_gbs = alg_bytes / (attn_ms * 1e-3) / 1e9
    if flops / alg_bytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        bound = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
                 "mfma_frac": round(achieved / peak, 4)}
    else:
        bound = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                 "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roofline = {**bound, "traffic": traffic, "algorithmic_bytes": round(alg_bytes),
                "kernel": ("attn_bwd_dkv + attn_bwd_dq + table-gradient sum" if args.backward and
                           args.rab else "attn_bwd_dkv + attn_bwd_dq" if args.backward else
                           "attn_fwd_mfma16" if case.dtype != "fp32" else "attn_fwd_mfma_f32") +
                          (" (graph replay, whole call)" if args.graph else ""),
                "kernel_ms": round(attn_ms, 5),
                "kernel_ms_median": round(kt.attn_median_ms, 5) if kt.calls else None,
                "kernel_ms_min": round(kt.attn_min_ms, 5) if kt.calls else None,
                # the shader clock the attention kernel's workgroups ran at in
                # the last timed call (null: no forward kernel timed)
                "clock_mhz_observed": round(kt.clock_mhz, 1) if kt.clock_mhz > 0 else None,
                "sched_kernel_ms": round(sched_ms, 5),
                "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}

    cpu = None
    if args.cpu_budget > 0:
        if args.cached:
            cpu = cpu_baseline_cached(cc, args.cpu_budget, rab=rab, hist_ts=hist_ts)
        elif args.backward:
            cpu = cpu_baseline_bwd(case, dout_host, args.cpu_budget, rab=rab)
        else:
            cpu = cpu_baseline(case, args.cpu_budget, rab=rab)

    L = case.lengths
    line = {
        "metric": ((METRIC_RAB_BWD if args.rab else METRIC_BWD) +
                   (" (target-aware mask)" if args.targets else "") if args.backward else
                   METRIC_RAB_CACHED if args.cached and args.rab else
                   METRIC_CACHED if args.cached else
                   METRIC_RAB_TARGETS if args.targets and args.rab else
                   METRIC_TARGETS if args.targets else
                   METRIC_DENSE if args.dense else
                   METRIC_RAB if args.rab else METRIC),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "clock_settle": {"calls": settle_calls, "seconds": round(settle_s, 3)},
        "higher_is_better": True,
        "scaling": "weak",
        # The pages time this shape only on other hardware (an Ascend NPU):
        # context, not a baseline of this run.
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_MFMA_TFLOPS["bf16"], 2),
        "config": {"workload": case.description, "num_seqs": case.num_seqs,
                   "total_tokens": case.total, "max_seq_len": int(L.max()), "heads": case.heads,
                   "d": case.d, "alpha": case.alpha, "n": case.n,
                   **({"candidates_per_seq": int(case.num_targets[0])} if args.targets else {}),
                   **({"cached_history_per_seq": int(cc.hist_lengths[0])} if args.cached else {}),
                   **({"layout": "(batch, heads, seq_len, d)"} if args.dense else {}),
                   **({"launch": "HIP graph replay"} if args.graph else {}),
                   **({"rab_positions": int(rab.pos_bias.size),
                       "rab_time_buckets": int(rab.time_bias.size)} if args.rab else {}),
                   "useful_gflop": round(flops / 1e9, 3)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
