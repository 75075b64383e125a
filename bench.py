#!/usr/bin/env python3
"""Benchmark of the chunked Gated DeltaNet forward on one MI355X.

One step = one la_gdn_fwd call (scheduler, intra-chunk pass with its fused
prologue, inter-chunk pass) over the varlen workload T = 4096, cu_seqlens =
[0, 1000, 2500, 4096], H = 16, K = V = 128, bf16, in-kernel q/k L2 norm,
zero initial state, output o and final states (the example call of the cuDNN
"Linear Attention" page).  Inputs are seeded synthetic tensors already
resident in HBM.  Steps rotate over several copies of the inputs, outputs and
workspaces (more bytes than the 256 MiB Infinity Cache holds), so each step
reads its operands from HBM rather than from the cache.

Prints one JSON line: tokens/s of the whole job, the roofline of one call (the
algorithmic bytes over the summed launch times of the call's kernels, each
from HIP events on the launch stream), and the fp64 CPU oracle timed on the
host cores as a baseline.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN fwd tokens/s (H=16,K=V=128,bf16) + % of MFMA/HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 64
WORKLOADS = {
    1: "tiny GDN fwd, T=256, one sequence, H=2, K=V=64, in-kernel q/k L2 norm, zero initial state, "
       "o + final state",
    2: "varlen GDN fwd, T=4096, cu_seqlens=[0,1000,2500,4096], H=16, K=V=128, in-kernel q/k L2 norm, "
       "zero initial state, o + final state",
    3: "dense batch GDN fwd, 8 x 4096 tokens, HK=4, HV=16, K=V=128, in-kernel q/k L2 norm, initial state, "
       "o + final state",
    4: "ragged long-context GDN fwd, 64 sequences of U[1,4096] tokens + one of 65536, H=32, K=V=128, "
       "in-kernel q/k L2 norm, zero initial state, o + final state",
    5: "GDN span summary, 32 spans x 8192 tokens, H=16, K=V=128, in-kernel k L2 norm, start state, "
       "end state + transition",
}
# options of the forward (la_gdn_fwd_ex), timed on a forward workload's shape
VARIANTS = {
    "plain": "",
    "fused": "beta as bf16 logits with the sigmoid in the kernel, and the safe gate "
             "-exp(a_log) softplus(g + dt_bias) from the raw gate",
    "series64": "with the state series every 64 tokens (bf16 rows)",
    "series64-fp32": "with the state series every 64 tokens (fp32 rows)",
    "gdp2": "Gated Delta Product, 2 Householder updates per token (k, v, beta update-major)",
    "summary-bwd": "the span summary's mirror for the state gradient (la_gdn_summary_bwd: output and "
                   "end-state gradients in, start-state gradient out)",
    "bwd": "the full backward (la_gdn_bwd: output and final-state gradients in; dq, dk, dv, dg, dbeta and "
           "the initial-state gradient out, fp32)",
    "bwd-series": "the full backward given the forward's fp32 state series every 64 tokens (la_gdn_bwd_ex: "
                  "the forward's state pass is not run again; the series is counted as read)",
}


def backward_counts(lengths, HK, HV, K, V, with_init):
    """Bytes and flops of the full backward (intermediates excluded).

    Bytes: q, k, v and the output gradient (bf16), g and beta (fp32) read; dq, dk, dv,
    dg and dbeta (fp32) written; per sequence and head the final-state gradient read,
    the initial-state gradient written and the initial state read when given.  Flops of
    the chunked method, masked tiles counted whole: the forward again (as
    algorithmic_counts), the reverse chunk pass (K dS, P^T dO, Q^T dO, W^T dU:
    2 (3 K V + C V) per token-head) and the intra pass (U, dO S0^T, dU S0^T, U dS^T:
    8 K V; eight 64 x 64 x K products, three 64 x 64 x V and two 64 x 64 x 64:
    2 C (8 K + 3 V + 2 C) per token-head)."""
    T = sum(lengths)
    N = len(lengths)
    C = CHUNK
    by = (T * (2 * HK * K * 2 + 2 * HV * V * 2 + 2 * HV * 4 + 2 * HK * K * 4 + HV * V * 4 + 2 * HV * 4)
          + N * HV * K * V * 4 * (2 + int(with_init)))
    _, fwd = algorithmic_counts(lengths, HK, HV, K, V, False, with_init, True)
    fl = fwd + T * HV * (2 * (3 * K * V + C * V) + 8 * K * V + 2 * C * (8 * K + 3 * V + 2 * C))
    return by, fl


def algorithmic_counts(lengths, HK, HV, K, V, summary, with_init, with_final, nh=1, beta_bytes=4,
                       series_bytes=0):
    """Bytes and flops the method must move and compute (intermediates excluded).

    Forward bytes: q, k (bf16, per qk-head), v, o (bf16, per v-head), g, beta
    (fp32 per v-head), plus the fp32 states read/written: 1032 bytes per
    token-head at H = 16, K = V = 128.  Forward flops: per qk-head token the two
    chunk Gram products (k k^T and q k^T, 2 * 2 C K); per v-head token the W / U~
    products, the masked P U_new, W S, Q S and the state update
    (2 (3 K V + C (K + 2 V))), 180,224 per token-head at H = 16, K = V = 128.
    Span summary: no q and no o; bytes add the start, end and transition states;
    flops are the k k^T Gram product, W, U~, W S and the state update for the
    widened state [S | P] (K x (V + K)): also 180,224 per token-head at
    K = V = 128.

    Forward options: beta_bytes = 2 for bf16 beta logits; series_bytes = the
    state series written; nh > 1 (Gated Delta Product) reads nh rows of k, v and
    beta per token, and its flops are those of the chunked method over the T nh
    update rows (the q rows of a token's other updates are zeros, and the masked
    tiles are counted whole as above)."""
    T = sum(lengths)
    N = len(lengths)
    C = CHUNK
    if summary:
        by = T * (HK * K * 2 + HV * V * 2 + 2 * HV * 4) + N * HV * 4 * (K * V * (int(with_init) + 1) + K * K)
        VA = V + K
        fl = T * (HK * 2 * C * K + HV * 2 * (C * (K + V) + 2 * K * VA))
    else:
        by = (T * (HK * K * 2 * (1 + nh) + HV * V * 2 * (nh + 1) + HV * (4 + beta_bytes * nh))
              + N * HV * K * V * 4 * (int(with_init) + int(with_final)) + series_bytes)
        fl = T * nh * (HK * 2 * 2 * C * K + HV * 2 * (3 * K * V + C * (K + 2 * V)))
    return by, fl


def measured_traffic(kernel_src: str, kernels):
    """HBM bytes of one call (FETCH_SIZE + WRITE_SIZE of each of its kernels, calibrated)
    from the committed counter record, or None when the kernel source changed since
    the counters were taken (the record is then stale and must be measured again)."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(rec_path))
        h = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != h:
        return None
    per = rec.get("kernels", {})
    if any(k not in per for k in kernels):
        return None
    return int(sum(1024 * (per[k]["fetch_kib"] * rec["fetch_scale"] + per[k]["write_kib"] * rec["write_scale"])
                   for k in kernels))


def host_cpu():
    """The host's logical CPU count, the CPUs this process may run on, and the CPU model."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return os.cpu_count() or 1, usable, model


def cpu_baseline(problem, min_seconds: float = 10.0, max_reps: int = 400):
    """The fp64 oracle over the whole workload (all 48 (sequence, head) units),
    on the host cores, repeated until about min_seconds of wall time (a bounded
    sample of CPU work, so that the default run still finishes in about a minute).
    The oracle runs on the host's CPU share of one GPU (16 threads, or fewer when
    fewer CPUs are usable); the host's CPU count and model are reported beside it."""
    import oracle
    o = oracle.Oracle(problem)
    nt = oracle.default_threads()
    o.run_units([(0, 0)], num_threads=1)   # load the library outside the timing
    reps = 0
    t0 = time.perf_counter()
    while True:
        o.run_all(num_threads=nt)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    ncpu, usable, model = host_cpu()
    return {"value": reps * problem.total_tokens / dt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "host_cpus": ncpu, "usable_cpus": usable, "cpu_model": model,
            "sample": f"the whole workload ({problem.num_seqs * problem.num_v_heads} (sequence, head) units, "
                      f"{problem.total_tokens} tokens, fp64 token recurrence) run {reps} times: "
                      f"{dt:.2f} s wall on {nt} threads ({usable} usable of {ncpu} logical CPUs, {model})"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="input/output sets rotated over (cache-cold steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="the workload timed: 2 (default) is the bench line; 1, 3, 4 (forward) and 5 (span "
                         "summary) report the same fields for the other configurations, with inputs drawn on "
                         "the device and no CPU baseline")
    ap.add_argument("--variant", default="plain", choices=sorted(VARIANTS),
                    help="forward options timed on the workload's shape (forward workloads only): "
                         + "; ".join(f"{k}: {v}" for k, v in VARIANTS.items() if v))
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--measure-copy", action="store_true",
                    help="also time a 1 GiB device-to-device copy (best of 5, events) and report its read + "
                         "write rate in path.copy_gbs: the streaming rate HBM gives in practice, beside the "
                         "8 TB/s peak the roofline fractions use")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences and heads are independent, so more GPUs would shard them with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import gated_delta_rule_50_amd as la
    from workloads import fused_problem, gdp_problem, make_problem

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    la.load_library()

    wl = args.workload
    variant = args.variant
    prob = make_problem(wl) if wl == 2 else make_problem(wl, device="cuda")
    summary = prob.summary
    if variant == "summary-bwd":
        if not summary:
            print("--variant summary-bwd applies to the span summary workload (5)", file=sys.stderr)
            return 2
    elif variant != "plain" and summary:
        print("--variant applies to the forward workloads (1 to 4)", file=sys.stderr)
        return 2
    if variant.startswith("bwd") and wl == 4:
        print("--variant bwd runs on the workloads 1, 2 and 3", file=sys.stderr)
        return 2
    lengths = prob.lengths()
    T, HK, HV, K, V = prob.total_tokens, prob.num_qk_heads, prob.num_v_heads, prob.head_dim_k, prob.head_dim_v
    N = prob.num_seqs
    # the variants draw their own inputs of the same shape (seeded by the workload number)
    gen_dev = "cpu" if wl == 2 else "cuda"
    with_init = prob.state is not None
    if variant == "fused":
        prob = fused_problem(lengths, HK, HV, K, V, seed=wl, with_state=with_init, device=gen_dev)
    elif variant == "gdp2":
        prob = gdp_problem(lengths, 2, HK, HV, K, V, seed=wl, with_state=with_init, device=gen_dev)
    nh = 2 if variant == "gdp2" else 1
    every = 64 if variant.startswith("series64") else 0
    ck_dtype = torch.float32 if variant == "series64-fp32" else torch.bfloat16
    n_ck = la.checkpoint_entries(prob.cu_seqlens, every) if every else 0
    count_kw = {"nh": nh, "beta_bytes": 2 if variant == "fused" else 4,
                "series_bytes": n_ck * HV * K * V * (4 if ck_dtype == torch.float32 else 2)}

    # one copy is enough once a copy alone is larger than the Infinity Cache
    by0, _ = algorithmic_counts(lengths, HK, HV, K, V, summary, with_init, True, **count_kw)

    def fresh_copy(pr):
        def cl(x):
            return None if x is None else x.to(dev).clone()
        return dataclasses.replace(pr, cu_seqlens=cl(pr.cu_seqlens), q=cl(pr.q), k=cl(pr.k), v=cl(pr.v),
                                   g=cl(pr.g), beta=cl(pr.beta), state=cl(pr.state), a_log=cl(pr.a_log),
                                   dt_bias=cl(pr.dt_bias))

    copies = max(1, args.copies) if by0 < (1 << 30) else 1
    sets = []
    bwd_in = None
    if variant.startswith("bwd"):
        gen = torch.Generator(device="cuda").manual_seed(wl)
        bwd_in = (torch.randn((T, HV, V), generator=gen, device=dev).to(torch.bfloat16),
                  torch.randn((N, HV, K, V), generator=gen, device=dev))
    if variant == "summary-bwd":
        gen = torch.Generator(device="cuda").manual_seed(wl)
        bwd_in = (torch.randn((T, HV, V), generator=gen, device=dev).to(torch.bfloat16),
                  torch.randn((N, HV, K, V), generator=gen, device=dev))
        prob = dataclasses.replace(prob, q=torch.randn(prob.k.shape, generator=gen, device=dev).to(torch.bfloat16))
    for ic in range(copies):
        g = fresh_copy(prob)
        if summary:
            out = torch.empty((N, HV, K, K), dtype=torch.float32, device=dev)   # transition
            desc = la.make_desc(g.k, g.v, g.g, g.beta, N)
        else:
            out = torch.empty((T, HV, V), dtype=torch.bfloat16, device=dev)
            desc = la.make_desc(g.k, g.v, g.g, g.beta, N, q=g.q, out=out, num_householder=nh)
        fin = torch.empty((N, HV, K, V), dtype=torch.float32, device=dev)
        if variant.startswith("bwd"):
            desc = la.make_desc(g.k, g.v, g.g, g.beta, N, q=g.q, out=bwd_in[0])
            ws = torch.empty(la.la_gdn_bwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)
            grads = {"dq": torch.empty((T, HK, K), device=dev), "dk": torch.empty((T, HK, K), device=dev),
                     "dv": torch.empty((T, HV, V), device=dev), "dg": torch.empty((T, HV), device=dev),
                     "dbeta": torch.empty((T, HV), device=dev), "d_initial_state": fin}
            series = None
            if variant == "bwd-series":
                # the forward's state series, made once before the timed region
                _, _, series = la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state,
                                                checkpoint_every_n_tokens=64, checkpoint_dtype=torch.float32)
            sets.append((g, grads, fin, ws, series))
            continue
        ws = torch.empty(la.la_gdn_workspace_bytes_ex(desc, summary, nh), dtype=torch.uint8, device=dev)
        ck = torch.empty((n_ck, HV, K, V), dtype=ck_dtype, device=dev) if every else None
        sets.append((g, out, fin, ws, ck))
    stream = torch.cuda.current_stream()

    def step(i):
        g, out, fin, ws, ck = sets[i % len(sets)]
        if variant.startswith("bwd"):
            la.la_gdn_bwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, bwd_in[0], initial_state=g.state,
                          d_final_state=bwd_in[1], workspace=ws, stream=stream, out=out, chunk_states=ck)
        elif variant == "summary-bwd":
            la.la_gdn_summary_bwd(g.q, g.k, g.g, g.beta, g.cu_seqlens, bwd_in[0], bwd_in[1], d_start_state=fin,
                                  workspace=ws, stream=stream)
        elif summary:
            la.la_gdn_summary(g.k, g.v, g.g, g.beta, g.cu_seqlens, start_state=g.state, end_state=fin,
                              transition=out, l2norm=True, workspace=ws, stream=stream)
        elif variant == "plain":
            la.la_gdn_fwd(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state, out=out,
                          final_state=fin, l2norm=True, workspace=ws, stream=stream)
        else:
            la.la_gdn_fwd_ex(g.q, g.k, g.v, g.g, g.beta, g.cu_seqlens, initial_state=g.state, out=out,
                             final_state=fin, l2norm=True, beta_sigmoid=g.beta_sigmoid, a_log=g.a_log,
                             dt_bias=g.dt_bias, checkpoint_every_n_tokens=every, checkpoints=ck,
                             num_householder=nh, workspace=ws, stream=stream)

    copy_gbs = None
    if args.measure_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        copy_gbs = 2 * (1 << 30) / (best * 1e-3) / 1e9
        del src, dst

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if la.la_gdn_device_status(sets[0][3]) != la.LA_DEVICE_OK:
        print("device status reports malformed cu_seqlens", file=sys.stderr)
        return 1

    # timed region: K steps between device synchronizations, nothing else enqueued
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # host time of one call (argument checks, workspace carving, two or three
    # launches, the Python binding): the calls are enqueued back to back and timed
    # on the host only
    torch.cuda.synchronize()
    n_host = min(args.steps, 50)
    h0 = time.perf_counter()
    for i in range(n_host):
        step(i)
    h1 = time.perf_counter()
    torch.cuda.synchronize()

    # second timed region of the same K steps with per-kernel HIP events recorded
    # by the library around each launch on the launch stream (the events add
    # their own gaps, so the throughput above comes from the clean region)
    la.la_gdn_profile_enable(True)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = {}
    for kid in range(la.LA_KERNEL_COUNT):
        ms, n = la.la_gdn_profile_read(kid)
        kern[la.la_gdn_kernel_name(kid)] = {"avg_us": 1e3 * ms / max(n, 1), "launches": n}
    la.la_gdn_profile_enable(False)

    elapsed = t1 - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = T * args.steps / elapsed

    by, fl = algorithmic_counts(lengths, HK, HV, K, V, summary, with_init, True, **count_kw)
    if variant == "summary-bwd":
        # q, k (bf16 per q/k head), d_out (bf16), g, beta per value head; the end- and
        # start-state gradients.  Flops of the chunked method: per q/k-head token the Gram
        # and q k^T products (2 * 2 C K), per value-head token W (2 C K) and the reverse
        # chunk pass (2 (3 K V + C V))
        by = T * (2 * HK * K * 2 + HV * V * 2 + 2 * HV * 4) + 2 * N * HV * K * V * 4
        fl = T * (HK * 2 * 2 * CHUNK * K + HV * (2 * CHUNK * K + 2 * (3 * K * V + CHUNK * V)))
    elif variant.startswith("bwd"):
        by, fl = backward_counts(lengths, HK, HV, K, V, with_init)
        if variant == "bwd-series":
            by += la.checkpoint_entries(prob.cu_seqlens, 64) * HV * K * V * 4
    # Roofline of the call: the path's algorithmic bytes (or flops) over the GPU time of
    # all the kernels one call launches, each timed with HIP events on the launch
    # stream (their sum is what rocprofv3 reports for the same kernels).  The span
    # summary sits at the ridge and is priced on bf16 MFMA flops.
    launched = [k for k, v in kern.items() if v["launches"] > 0]
    call_us = sum(kern[k]["avg_us"] for k in launched)
    step_s = ms_per_step * 1e-3
    if summary and variant != "summary-bwd":
        roof = {"bound": "mfma", "achieved": fl / (call_us * 1e-6) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / (call_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # measured HBM bytes of the call's kernels (the committed counter record covers the
    # default workload only)
    roof["traffic"] = (measured_traffic(os.path.join(ROOT, "gated_delta_rule_50_amd", "csrc", "la_gdn_kernels.hip"),
                                        launched) if wl == 2 and variant == "plain" else None)
    roof.update({"kernel": " + ".join(launched) + " (one call)", "algorithmic_bytes_per_launch": by,
                 "algorithmic_flops_per_launch": fl, "avg_launch_us": call_us,
                 "kernel_avg_us": {k: kern[k]["avg_us"] for k in launched}})

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[wl] + (f"; {VARIANTS[variant]}" if VARIANTS[variant] else ""),
                   "T": T, "N": N, "HK": HK, "HV": HV, "K": K, "V": V, "copies_rotated": len(sets),
                   "global_batch": N, "seq_len": T, "parallelism": "single GPU"},
        "roofline": roof,
        "path": {"algorithmic_bytes": by, "algorithmic_flops": fl,
                 "token_heads_per_s": value * HV,
                 "host_us_per_call": 1e6 * (h1 - h0) / n_host,
                 "hbm_frac": by / step_s / (HBM_PEAK_GBS * 1e9),
                 "mfma_frac": fl / step_s / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                 "kernels": kern},
    }
    if copy_gbs is not None:
        rec["path"]["copy_gbs"] = copy_gbs
    if not args.no_cpu_baseline and wl == 2 and variant == "plain":
        rec["cpu_baseline"] = cpu_baseline(prob)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
