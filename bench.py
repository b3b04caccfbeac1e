#!/usr/bin/env python3
"""Benchmark: one step = forward + backward of fused feature-map linear
attention over one batch of seeded synthetic input, on one MI355X.

    python bench.py [--gpus 1] [--steps K=30] [--warmup W] [--workload NAME]
                    [--dtype bf16|f32] [--mode causal|bidir] [--no-flush]

NAME is an attention workload of seeded_inputs.WORKLOADS, the materialised
GQA op (seeded_inputs.GQA_OPS: expand + reduce per step) or the low-rank
projection (seeded_inputs.LOWRANK_OPS: fwd + bwd per step); --dtype / --mode
pick among a workload's storage types and modes (default: its first).

Default workload: causal, bf16 storage, B=2, H=32, N=16384, D=128, elu+1,
eps=1e-6 (q, k, v ~ 0.5 N(0,1), grad_out ~ N(0,1), seed 0).  Inputs, outputs
and workspaces are resident in HBM before timing.  W untimed steps (default: as
many as fill 0.5 s), then K timed steps, each preceded (outside its timing) by
a read of a 1 GiB buffer that evicts the L2 and last-level caches, and each
bracketed by a pair of HIP events on the stream the library launches on; the
K steps are bracketed by device synchronisations.  value = tokens / median
step time.  Further passes of K flushed steps give the per-kernel breakdown
(the library's own launch events), the forward alone (la_fwd, with its own
roofline fraction) and the step with the backward recomputing the state (la_bwd).  The
forward and the backward of a step share one workspace, so the backward reuses
the forward's state records (la_bwd_saved, as the autograd form does).  One
JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix
FP32_PEAK_TFLOPS = 157.3        # MI355X fp32 (vector and matrix)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_bytes(name, w, s):
    """Algorithmic HBM bytes of one launch of kernel ``name``: the tensors it
    must read and write for the part of the method it computes (workspace
    records excluded).  q-sized = B*H*N*D*s, kv-sized = B*H_kv*N*D*s."""
    qb = w.B * w.H * w.N * w.D * s
    kvb = w.B * w.Hkv * w.N * w.D * s
    rows = w.B * w.H * w.N * 4            # one float per query row (den or c)
    table = {
        "state": 2 * kvb,                                 # k, v
        "fwd_causal": 2 * qb + 2 * kvb,                   # q, k, v -> out
        "fwd_bidir": 2 * qb,                              # q -> out
        "bwd_q_causal": 3 * qb + 2 * kvb + 2 * rows,      # q, k, v, g -> dq, den, c
        "bwd_q_bidir": 3 * qb,                            # q, g -> dq
        "bwd_kv_causal": 2 * qb + 4 * kvb + 2 * rows,     # q, g, den, c, k, v -> dk, dv
        "bwd_kv_bidir": 4 * kvb,                          # k, v -> dk, dv
        "bwd_r": 2 * qb + 2 * rows,                       # q, g, den, c (per-segment R, r)
    }
    # matrix-core kernels compute the same parts of the method
    alias = {"k_state_mfma": "state", "k_fwd_mfma": "fwd_causal", "k_fwd_split_mfma": "fwd_causal",
             "k_bwd_q_mfma": "bwd_q_causal",
             "k_bwd_kv_mfma": "bwd_kv_causal", "k_fwd_bidir_mfma": "fwd_bidir",
             "k_bwd_q_bidir_mfma": "bwd_q_bidir", "k_bwd_kv_bidir_mfma": "bwd_kv_bidir",
             "k_bwd_q_cos_mfma": "bwd_q_causal", "k_bwd_r_cos_mfma": "bwd_r",
             "k_bwd_kv_cos_mfma": "bwd_kv_causal", "k_bwd_q_cos_bidir_mfma": "bwd_q_bidir",
             "k_bwd_r_cos_bidir_mfma": "bwd_r", "k_bwd_kv_cos_bidir_mfma": "bwd_kv_bidir",
             "k_state_f32": "state",
             "k_fwd_bidir_f32": "fwd_bidir", "k_bwd_q_bidir_f32": "bwd_q_bidir",
             "k_bwd_kv_bidir_f32": "bwd_kv_bidir"}
    if name in alias:
        return table[alias[name]]
    for key, val in table.items():
        if name.endswith(key):
            return val
    return None


def measured_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed counter summary
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size), or None
    when there is no summary or a kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    srcdir = os.path.join(ROOT, "linear_attention_transformers_amd", "csrc")
    for line in text.splitlines():
        if line.startswith("Kernel sources (sha256 prefix):"):
            for item in line.split(":", 1)[1].split(","):
                name, digest = item.strip().split("=")
                cur = hashlib.sha256(open(os.path.join(srcdir, name), "rb").read()).hexdigest()
                if not cur.startswith(digest):
                    return None
    scale, rows = None, {}
    for line in text.splitlines():
        parts = line.split()
        if len(parts) == 4 and parts[0] == "fetch_scale":
            scale = (float(parts[1]), float(parts[3]))
        elif len(parts) == 3 and parts[0].startswith("k_"):
            rows[parts[0]] = (float(parts[1]), float(parts[2]))
    if scale is None or kernel not in rows:
        return None
    fetch, write = rows[kernel]
    return (fetch * scale[0] + write * scale[1]) * 1024.0


def traffic_key(name, dtype, mode):
    """Name of the counter summary of a workload variant (profiles/counters_<key>.md)."""
    import seeded_inputs as si
    w = si.WORKLOADS[name]
    if dtype == w.dtypes[0] and mode == w.modes[0]:
        return name
    return "%s_%s_%s" % (name, dtype, mode)


def step_roofline(w, s, causal):
    """Time of one step (fwd+bwd, or fwd for a forward-only workload) at the
    roofline: each pass at the larger of its algorithmic bytes at HBM peak and
    its algorithmic flops (state updates and reads, 2*F*D per token each;
    F = 2D with cos/sin) at the matrix peak of the storage type (bf16, or
    float32 for float32 storage), the two passes summed."""
    br = 2 if w.cos else 1
    tokD = w.B * w.N * w.D
    fwd_bytes = s * tokD * (2 * w.H + 2 * w.Hkv) + (8 * w.N if w.cos else 0)
    bwd_bytes = s * tokD * (3 * w.H + 4 * w.Hkv)
    fwd_flops = br * 2 * w.D * w.D * w.B * w.N * (w.H + w.Hkv)
    bwd_flops = br * 2 * w.D * w.D * w.B * w.N * (3 * w.H + 3 * w.Hkv)
    if not w.backward:   # forward-only workload
        bwd_bytes = bwd_flops = 0
    peak = (BF16_PEAK_TFLOPS if s == 2 else FP32_PEAK_TFLOPS) * 1e12
    t = (max(fwd_bytes / (HBM_PEAK_GBS * 1e9), fwd_flops / peak) +
         max(bwd_bytes / (HBM_PEAK_GBS * 1e9), bwd_flops / peak))
    return t, fwd_bytes + bwd_bytes, fwd_flops + bwd_flops


def cpu_baseline(w, tensors, causal, budget_heads=None, min_seconds=10.0):
    """The CPU oracle, as it is, on whole (batch, KV head) groups at full N,
    fwd + bwd; throughput scaled to the whole workload by group count."""
    import numpy as np

    import oracle
    import seeded_inputs as si

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n_groups = w.B * w.Hkv
    nrep = w.H // w.Hkv
    take = budget_heads or max(1, threads // nrep)
    take = min(take, n_groups)
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)][:take]
    f64 = {n: si.exact_f64(t) for n, t in tensors.items() if t is not None and t.dim() == 4}
    parts = [oracle.group_slice(f64["q"], f64["k"], f64["v"], f64.get("grad_out"), b, g)
             for b, g in units]
    q = np.concatenate([p[0] for p in parts])
    k = np.concatenate([p[1] for p in parts])
    v = np.concatenate([p[2] for p in parts])
    g = np.concatenate([p[3] for p in parts]) if w.backward else None
    cw = sw = None
    if tensors.get("cos_weight") is not None:
        cw, sw = si.exact_f64(tensors["cos_weight"]), si.exact_f64(tensors["sin_weight"])
    kw = dict(is_causal=causal, phi=w.phi, eps=w.eps, cos_weight=cw, sin_weight=sw)
    # repeat the sample until about min_seconds of oracle time have passed
    reps, total = 0, 0.0
    while reps == 0 or (total < min_seconds and reps < 64):
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, **kw)
        if w.backward:
            oracle.bwd(q, k, v, g, **kw)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    t_full = dt * n_groups / take
    return {
        "value": w.B * w.N / t_full,
        "unit": "tokens/s",
        "cores": min(threads, take * nrep),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "%d of %d (batch, KV head) groups (%d query heads each) at full N=%d, "
                  "%s in fp64, mean of %d runs (%.1f s in all); scaled by group count"
                  % (take, n_groups, nrep, w.N, "fwd+bwd" if w.backward else "fwd", reps, total),
    }


def gqa_cpu_baseline(c, arrays, min_seconds=10.0):
    """The GQA oracle as it is (float64, NumPy) on one KV slab of k and its
    n_rep gradient slabs at full N; scaled to the op by slab count (2 B H_kv)."""
    from oracle import gqa as og

    nrep = c["H"] // c["Hkv"]
    k = arrays["k"][0:1, 0:1].astype(np.float64)
    gk = arrays["grad_k"][0:1, 0:nrep].astype(np.float64)
    reps, total = 0, 0.0
    while reps == 0 or (total < min_seconds and reps < 64):
        t0 = time.perf_counter()
        og.round_to(og.expand(k, nrep), c["dtype"])
        og.round_to(og.reduce(gk, nrep), c["dtype"])
        total += time.perf_counter() - t0
        reps += 1
    t_full = total / reps * 2 * c["B"] * c["Hkv"]
    return {"value": c["B"] * c["N"] / t_full, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "one KV slab of k (N=%d, D=%d) expanded to %d heads and its %d gradient "
                      "slabs summed, fp64 NumPy, mean of %d runs (%.1f s in all); scaled by the "
                      "op's %d slabs" % (c["N"], c["D"], nrep, nrep, reps, total,
                                          2 * c["B"] * c["Hkv"])}


def bench_gqa(args, name):
    """One step = la_gqa_expand (k, v) + la_gqa_reduce (grad_k, grad_v) on
    resident buffers; the same JSON fields as the attention workloads."""
    import ctypes

    import torch

    import linear_attention_transformers_amd as la
    import seeded_inputs as si

    c = si.GQA_OPS[name]
    B, H, Hkv, N, D = c["B"], c["H"], c["Hkv"], c["N"], c["D"]
    s = 2 if c["dtype"] == "bf16" else 4
    code = la.LA_BF16 if c["dtype"] == "bf16" else la.LA_F32
    lib = la.load_library()
    log("bench: drawing %s inputs" % name)
    arrays = si.gqa_draw(B, H, Hkv, N, D)
    t = si.to_torch(arrays, c["dtype"], "cuda")
    ko = torch.empty((B, H, N, D), dtype=t["k"].dtype, device="cuda")
    vo = torch.empty_like(ko)
    gk = torch.empty_like(t["k"])
    gv = torch.empty_like(t["v"])
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("bench: calibration copy of %d MiB done" % args.calibration_copy_mib)

    def step():
        st = lib.la_gqa_expand(P(t["k"]), P(t["v"]), P(ko), P(vo), B, Hkv, H, N, D, code, stream)
        st = st or lib.la_gqa_reduce(P(t["grad_k"]), P(t["grad_v"]), P(gk), P(gv), B, Hkv, H, N, D,
                                     code, stream)
        if st:
            raise RuntimeError(lib.la_last_error().decode())

    flush = None if args.no_flush else Flusher(torch.device("cuda:0"))
    args.warmup = warm_up(step, args.warmup, flush)
    log("bench: %d warmup steps done; %d timed steps" % (args.warmup, args.steps))
    step_ms, wall = timed_steps(step, args.steps, flush)
    st = stats(step_ms)
    la.timing_enable(True)
    try:
        timed_steps(step, args.steps, flush)
    finally:
        la.timing_enable(False)
    ktimes = la.timing_collect()
    kvb, qb = B * Hkv * N * D * s, B * H * N * D * s
    per_launch = {"k_gqa_expand": 2 * kvb + 2 * qb, "k_gqa_reduce": 2 * qb + 2 * kvb}
    dom_name, (launches, total_ms) = max(ktimes.items(), key=lambda kv: kv[1][1])
    avg_s = total_ms / launches / 1e3
    nbytes = per_launch[dom_name]
    ms_step = st["median_ms"]
    step_bytes = sum(per_launch.values())
    t_roof = step_bytes / (HBM_PEAK_GBS * 1e9)
    result = {
        "metric": "GQA expand+reduce tokens/sec and %% roofline, %s" % name,
        "value": B * N / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c["dtype"], "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "H_kv": Hkv, "N": N, "D": D,
                   "storage": c["dtype"], "pass": "expand (k, v) + reduce (grad_k, grad_v)"},
        "timing": dict(st, basis="median of per-step HIP events", flushed=flush is not None,
                       wall_s_incl_flushes=wall),
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": nbytes / avg_s / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nbytes / avg_s / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name, dom_name), "avg_launch_ms": avg_s * 1e3,
                     "algorithmic_bytes_per_launch": nbytes},
        "step_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_step,
                          "algorithmic_bytes": step_bytes, "algorithmic_flops": 0},
        "kernels_ms_per_step": {k: v[1] / args.steps for k, v in ktimes.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        result["cpu_baseline"] = gqa_cpu_baseline(c, arrays)
    print(json.dumps(result), flush=True)


def lowrank_cpu_baseline(c, arrays, min_seconds=10.0):
    """The low-rank oracle as it is (float64 NumPy) on a bounded row sample,
    fwd + bwd; throughput scaled to all M rows (every product is linear in M)."""
    from oracle import lowrank as olr

    rows = 1024
    x, U, V = (arrays[k].astype(np.float64) for k in ("x", "U", "V"))
    b, g = arrays["bias"].astype(np.float64), arrays["grad_out"].astype(np.float64)
    xs, gs = x[:rows], g[:rows]
    reps, total = 0, 0.0
    while reps == 0 or (total < min_seconds and reps < 64):
        t0 = time.perf_counter()
        olr.fwd(xs, U, V, b)
        olr.bwd(xs, U, V, gs, b)
        total += time.perf_counter() - t0
        reps += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": rows / (total / reps), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows, fwd+bwd in fp64 NumPy (BLAS threads), mean of %d runs "
                      "(%.1f s in all); rows scale linearly" % (rows, c["M"], reps, total)}


def bench_lowrank(args, name):
    """One step = la_lowrank_fwd + la_lowrank_bwd on resident buffers."""
    import ctypes

    import torch

    import linear_attention_transformers_amd as la
    import seeded_inputs as si

    c = si.LOWRANK_OPS[name]
    M, n_in, rank, n_out = c["M"], c["n_in"], c["rank"], c["n_out"]
    lib = la.load_library()
    log("bench: drawing %s inputs" % name)
    arrays = si.lowrank_draw(M, n_in, rank, n_out)
    t = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16).contiguous() for k, v in arrays.items()}
    y = torch.empty((M, n_out), dtype=torch.bfloat16, device="cuda")
    gx, gU, gV, gb = (torch.empty_like(t[k]) for k in ("x", "U", "V", "bias"))
    wsb = int(lib.la_lowrank_workspace_bytes(la.LA_OP_BWD, M, n_in, rank, n_out, la.LA_BF16))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    P = lambda x: ctypes.c_void_p(x.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        st = lib.la_lowrank_fwd(P(t["x"]), P(t["U"]), P(t["V"]), P(t["bias"]), P(y), M, n_in, rank, n_out,
                                la.LA_BF16, P(ws), wsb, stream)
        st = st or lib.la_lowrank_bwd(P(t["x"]), P(t["U"]), P(t["V"]), P(t["grad_out"]), P(gx), P(gU), P(gV),
                                      P(gb), M, n_in, rank, n_out, la.LA_BF16, P(ws), wsb, stream)
        if st:
            raise RuntimeError(lib.la_last_error().decode())

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = None if args.no_flush else Flusher(torch.device("cuda:0"))
    args.warmup = warm_up(step, args.warmup, flush, sync_every=4)
    log("bench: %d warmup steps done; %d timed steps" % (args.warmup, args.steps))
    step_ms, wall = timed_steps(step, args.steps, flush)
    st = stats(step_ms)
    la.timing_enable(True)
    try:
        timed_steps(step, args.steps, flush)
    finally:
        la.timing_enable(False)
    ktimes = la.timing_collect()
    mnk = 2.0 * M * rank   # flops of one product per unit of its third size
    flops = {"k_lowrank_gemm_xVt": mnk * n_in, "k_lowrank_gemm_tUt": mnk * n_out,
             "k_lowrank_gemm_gU": mnk * n_out, "k_lowrank_gemm_gtV": mnk * n_in,
             "k_lowrank_gemm_gTt": mnk * n_out, "k_lowrank_gemm_gtTx": mnk * n_in}
    gemms = {k: v for k, v in ktimes.items() if k in flops}
    dom_name, (launches, total_ms) = max(gemms.items(), key=lambda kv: kv[1][1])
    avg_s = total_ms / launches / 1e3
    ms_step = st["median_ms"]
    step_flops = mnk * (n_in + n_out) + mnk * (n_in + 2 * n_out + 2 * n_in)   # fwd 2, bwd 5 products
    step_bytes = 2 * (2 * M * n_in + 2 * M * n_out + 2 * rank * (n_in + n_out) + 2 * n_out)   # x, y, g, gx, U, V, grads
    t_roof = max(step_flops / (BF16_PEAK_TFLOPS * 1e12), step_bytes / (HBM_PEAK_GBS * 1e9))
    ach = flops[dom_name] / avg_s / 1e12
    result = {
        "metric": "low-rank projection fwd+bwd tokens/sec and %% roofline, %s" % name,
        "value": M / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "M": M, "n_in": n_in, "rank": rank, "n_out": n_out, "bias": True,
                   "storage": "bf16", "pass": "fwd + bwd (bwd recomputes t)"},
        "timing": dict(st, basis="median of per-step HIP events", flushed=flush is not None,
                       wall_s_incl_flushes=wall),
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(name, dom_name), "avg_launch_ms": avg_s * 1e3,
                     "algorithmic_flops_per_launch": flops[dom_name]},
        "step_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_step,
                          "algorithmic_bytes": step_bytes, "algorithmic_flops": step_flops},
        "kernels_ms_per_step": {k: v[1] / args.steps for k, v in ktimes.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        result["cpu_baseline"] = lowrank_cpu_baseline(c, arrays)
    print(json.dumps(result), flush=True)


class Flusher:
    """Evicts the L2 and last-level caches between timed steps by reading a
    1 GiB buffer (larger than both).  A read, not a write: the lines it leaves
    are clean, whereas the dirty lines of a write would be written back inside
    the next timed step (a 1 GiB write just before a 512 MiB streaming read
    slowed that read by about 40% on the box).  Dirty output of the previous
    step is written back during this read, outside the timed window."""

    def __init__(self, dev, mib=1024):
        import torch
        self.buf = torch.zeros((mib << 20) // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.amax(self.buf, dim=0, out=self.out)


def warm_up(step, warmup, flush, sync_every=8):
    """W untimed steps in the timed steps' own pattern: each after a cache
    flush when the timed steps flush, so the timed steps start at the device's
    steady state for that pattern (after unflushed warm-up steps, the first
    dozen or so flushed steps of the headline ran up to 30% slower).
    warmup None: as many as fill 0.5 s (at least 3).  Returns W."""
    import torch
    n, t_w = 0, time.perf_counter()
    while (n < 3 or time.perf_counter() - t_w < 0.5) if warmup is None else n < warmup:
        if flush is not None:
            flush()
        step()
        n += 1
        if n % sync_every == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def timed_steps(step, K, flush):
    """Per-step times (ms) of K calls of step(), each bracketed by HIP events
    on the current stream, each preceded by flush() (if given) outside the
    events; the K steps are bracketed by device synchronisations."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [e0.elapsed_time(e1) for e0, e1 in evs], wall


def stats(ms):
    v = sorted(ms)
    return {"median_ms": v[len(v) // 2], "min_ms": v[0], "mean_ms": sum(v) / len(v),
            "max_ms": v[-1], "n": len(v)}


def calibrate(dev, flush):
    """Achievable peaks measured on this device (flushed, median of 5): a
    512 MiB device copy (read + write bytes), a 1 GiB reduction (read bytes)
    and a bf16 GEMM 8192^3 (the vendor library), beside the spec figures."""
    import torch
    src = torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    red = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev)
    o = torch.empty((), dtype=torch.float32, device=dev)
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    c = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        dst.copy_(src)
        torch.amax(red, dim=0, out=o)
        torch.matmul(a, b, out=c)
    cp, _ = timed_steps(lambda: dst.copy_(src), 5, flush)
    rd, _ = timed_steps(lambda: torch.amax(red, dim=0, out=o), 5, flush)
    mm, _ = timed_steps(lambda: torch.matmul(a, b, out=c), 5, flush)
    med = lambda x: sorted(x)[len(x) // 2] / 1e3
    res = {"copy_gbs": 2 * src.numel() * 4 / med(cp) / 1e9,
           "read_gbs": red.numel() * 4 / med(rd) / 1e9,
           "bf16_gemm_tflops": 2 * 8192 ** 3 / med(mm) / 1e12,
           "spec_hbm_gbs": HBM_PEAK_GBS, "spec_bf16_tflops": BF16_PEAK_TFLOPS,
           "how": "flushed, median of 5: torch copy of 512 MiB (read+write bytes), "
                  "torch amax over 1 GiB (read bytes), torch bf16 matmul 8192^3"}
    del src, dst, red, a, b, c
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def fwd_roofline(w, s):
    """Time of one la_fwd at the roofline: q, k, v read and out written once
    at HBM peak vs the state reads and updates (2 F D per query token and per
    key token) at the matrix peak."""
    br = 2 if w.cos else 1
    tokD = w.B * w.N * w.D
    nbytes = s * tokD * (2 * w.H + 2 * w.Hkv) + (8 * w.N if w.cos else 0)
    flops = br * 2 * w.D * w.D * w.B * w.N * (w.H + w.Hkv)
    peak_f = BF16_PEAK_TFLOPS if s == 2 else FP32_PEAK_TFLOPS
    return max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (peak_f * 1e12)), nbytes, flops


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # default: as many steps as fill 0.5 s (at least 3): the GPU's clocks ramp
    # up over the first tenths of a second of load, and a short warm-up would
    # time the ramp; the count used is reported
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dtype", default=None, choices=("bf16", "f32"))
    ap.add_argument("--mode", default=None, choices=("causal", "bidir"))
    ap.add_argument("--no-flush", action="store_true",
                    help="time back-to-back steps with warm caches (for comparison)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before warmup, copy a buffer of this many MiB once (a plain "
                         "device copy of known size, to scale HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_transformers_amd as la
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    la.load_library()
    name = args.workload or si.HEADLINE
    if name in si.GQA_OPS:
        return bench_gqa(args, name)
    if name in si.LOWRANK_OPS:
        return bench_lowrank(args, name)
    w = si.WORKLOADS[name]
    dtype = args.dtype or w.dtypes[0]
    mode = args.mode or w.modes[0]
    if dtype not in w.dtypes or mode not in w.modes:
        print("workload %s has storage %s and modes %s" % (name, w.dtypes, w.modes), file=sys.stderr)
        sys.exit(2)
    causal = mode == "causal"
    s = 2 if dtype == "bf16" else 4
    dev = torch.device("cuda:0")

    log("bench: drawing %s inputs (%s, %s)" % (name, dtype, mode))
    t = si.workload_inputs(w, dtype, dev)
    cw, sw = t["cos_weight"], t["sin_weight"]
    out = torch.empty_like(t["q"])
    grads = (torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"]))
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    # one workspace for the forward and the backward: the backward reuses the
    # forward's state records (la_bwd_saved), as the autograd form does
    ws = torch.empty(la.workspace_bytes("bwd" if w.backward else "fwd", w.B, w.H, w.Hkv, w.N, w.D,
                                        code, causal, w.cos), dtype=torch.uint8, device=dev)
    flush = None if args.no_flush else Flusher(dev)

    def fwd():
        la.fwd(t["q"], t["k"], t["v"], is_causal=causal, phi=w.phi, eps=w.eps, cos_weight=cw,
               sin_weight=sw, out=out, workspace=ws)

    def step(saved=True):
        fwd()
        if w.backward:
            la.bwd(t["q"], t["k"], t["v"], t["grad_out"], is_causal=causal, phi=w.phi,
                   eps=w.eps, cos_weight=cw, sin_weight=sw, workspace=ws, grads=grads,
                   state_from_fwd=saved)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("bench: calibration copy of %d MiB done" % args.calibration_copy_mib)

    args.warmup = warm_up(step, args.warmup, flush)
    log("bench: %d warmup steps done" % args.warmup)

    # A: the headline: per-step events only
    log("bench: %d timed steps%s" % (args.steps, "" if flush else " (no flush)"))
    step_ms, wall = timed_steps(step, args.steps, flush)
    st = stats(step_ms)
    tokens = w.B * w.N
    ms_step = st["median_ms"]
    value = tokens / (ms_step / 1e3)

    # B: per-kernel breakdown from the library's own launch events
    log("bench: %d steps with per-kernel events" % args.steps)
    la.timing_enable(True)
    try:
        timed_steps(step, args.steps, flush)
    finally:
        la.timing_enable(False)
    ktimes = la.timing_collect()

    # C: the forward alone
    log("bench: %d forward-only steps" % args.steps)
    fwd_ms, _ = timed_steps(fwd, args.steps, flush)
    fst = stats(fwd_ms)
    t_froof, f_bytes, f_flops = fwd_roofline(w, s)

    # D: the backward computing the state records again (la_bwd)
    recompute = None
    if w.backward:
        log("bench: %d steps with the backward recomputing the forward's state" % args.steps)
        rms, _ = timed_steps(lambda: step(saved=False), args.steps, flush)
        rst = stats(rms)
        recompute = dict(rst, value=tokens / (rst["median_ms"] / 1e3), unit="tokens/s")

    # dominant kernel by total event time over pass B
    dom_name, (launches, total_ms) = max(ktimes.items(), key=lambda kv: kv[1][1])
    avg_s = total_ms / launches / 1e3
    nbytes = kernel_bytes(dom_name, w, s)
    roof = {"bound": "hbm", "kernel": dom_name, "achieved": None, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": None, "traffic": measured_traffic(traffic_key(name, dtype, mode), dom_name),
            "avg_launch_ms": avg_s * 1e3, "algorithmic_bytes_per_launch": nbytes}
    if nbytes is not None:
        ach = nbytes / avg_s / 1e9
        roof["achieved"] = ach
        roof["frac"] = ach / HBM_PEAK_GBS
    t_roof, step_bytes, step_flops = step_roofline(w, s, causal)
    matrix = any("mfma" in k or k.endswith("_f32") for k in ktimes)
    mpeak = BF16_PEAK_TFLOPS if s == 2 else FP32_PEAK_TFLOPS
    fwd_kernels = [k for k in ktimes if not (k.startswith("k_bwd") or k == "k_scan_R")]

    calib = None
    if not args.no_calibration:
        log("bench: calibration (copy, read, bf16 GEMM)")
        calib = calibrate(dev, flush or Flusher(dev))
        if roof["achieved"] is not None:
            roof["frac_of_measured_copy"] = roof["achieved"] / calib["copy_gbs"]

    result = {
        "metric": ("fwd+bwd tokens/sec and % roofline, causal bf16 N=16384 D=128" if name == si.HEADLINE
                   and dtype == "bf16" and causal
                   else "%s tokens/sec and %% roofline, %s %s %s" % (
                       "fwd+bwd" if w.backward else "fwd", name, dtype, mode)),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s == 2 else "f32",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "N": w.N, "D": w.D,
                   "phi": w.phi, "causal": causal, "cos_sin": w.cos, "storage": dtype,
                   "eps": w.eps, "pass": "fwd+bwd" if w.backward else "fwd",
                   "bwd_state": "saved by the forward (la_bwd_saved)" if w.backward else None},
        "timing": dict(st, basis="median of per-step HIP events",
                       flushed=flush is not None, wall_s_incl_flushes=wall),
        "roofline": roof,
        "step_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms_step,
                          "algorithmic_bytes": step_bytes, "algorithmic_flops": step_flops},
        "fwd_roofline": {"t_roof_ms": t_froof * 1e3, "ms": fst["median_ms"],
                         "min_ms": fst["min_ms"], "frac": t_froof * 1e3 / fst["median_ms"],
                         "algorithmic_bytes": f_bytes, "algorithmic_flops": f_flops,
                         "kernels": fwd_kernels},
        "kernels_ms_per_step": {k: v[1] / args.steps for k, v in ktimes.items()},
        # algorithmic bytes of each kernel (as for roofline.achieved) over its
        # average launch time, and the step's algorithmic flops over the step
        # time against the peak of the units that run them
        "kernels_gbs": {k: kernel_bytes(k, w, s) / (v[1] / v[0] / 1e3) / 1e9
                        for k, v in ktimes.items() if v[0] and kernel_bytes(k, w, s) is not None},
        "matrix": {"achieved": step_flops / (ms_step / 1e3) / 1e12,
                   "peak": mpeak, "unit": "TFLOP/s",
                   "frac": step_flops / (ms_step / 1e3) / 1e12 / mpeak,
                   "units": ("%s matrix cores" % ("bf16" if s == 2 else "float32")) if matrix
                            else "float32 vector ALU"},
        "calibration": calib,
        "bwd_recomputing_state": recompute,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, t, causal)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
