"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the CPU oracle on the same seeded inputs, compare normwise.

Tolerances: 1e-4 for float32 storage, 2e-2 for bfloat16 storage with float32
accumulation, applied two ways to every output tensor:

* whole tensor: max |gpu - oracle| / max |oracle|;
* per block: the same ratio over each (batch, head, block of ``BLOCK`` rows),
  with the block's own max |oracle| as the scale (floored at ``FLOOR`` times
  the tensor's, so that blocks of exact zeros stay well defined).  Causal
  outputs shrink along the sequence (rows average over ever more values), so
  the whole-tensor ratio is set by the first rows and cannot see an error
  confined to late rows, such as a segment missing from later prefixes;
  the per-block ratio sees each block at its own scale.

With PARITY_LOG set to a file name, every comparison appends one JSON line
(label, per-tensor whole and worst-block errors, tolerance) to it.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest

import oracle
import seeded_inputs as si

TOL = {"f32": 1e-4, "bf16": 2e-2}
BLOCK = 512      # rows per block of the per-block gate
FLOOR = 1e-3     # block scale floor, relative to the tensor's max |oracle|


def gpu_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import linear_attention_transformers_amd as la
    la.load_library()   # raises (fails the test) if the HIP library is missing
    return torch, la


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0)) if b.size else 0.0


def block_rel(a, b, block=BLOCK, floor=FLOOR):
    """Worst per-block normwise error of a against b, both [..., N, D]: over
    every leading index and every block of ``block`` rows,
    max |a - b| / max(max |b| in the block, floor * max |b|)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    N = b.shape[-2]
    scale_all = float(np.max(np.abs(b)))
    a2 = a.reshape(-1, N, b.shape[-1])
    b2 = b.reshape(-1, N, b.shape[-1])
    worst = 0.0
    for r0 in range(0, N, block):
        d = np.max(np.abs(a2[:, r0:r0 + block] - b2[:, r0:r0 + block]), axis=(1, 2))
        m = np.max(np.abs(b2[:, r0:r0 + block]), axis=(1, 2))
        den = np.maximum(m, floor * scale_all)
        den = np.where(den > 0, den, 1.0)
        worst = max(worst, float(np.max(d / den)))
    return worst


def make(B, H, Hkv, N, D, dtype, scale=1.0, cos=False, seed=0, grad=True, device="cuda"):
    arrays = si.draw(B, H, Hkv, N, D, scale, seed, grad=grad)
    t = si.to_torch(arrays, dtype, device)
    if cos:
        import torch
        c, s = si.cos_sin(N)
        t["cos_weight"] = torch.from_numpy(c).to(device)
        t["sin_weight"] = torch.from_numpy(s).to(device)
    else:
        t["cos_weight"] = t["sin_weight"] = None
    return t


def np64(t):
    return None if t is None else si.exact_f64(t)


def run_gpu(la, t, causal, phi, eps=1e-6, seg_len=0, backward=True, saved=False):
    """la_fwd, then (backward) la_bwd; saved=True gives both one workspace and
    runs the backward on the forward's state records (la_bwd_saved), the
    path the benchmark times."""
    ws = None
    if saved:
        import torch
        q = t["q"]
        B, H, N, D = q.shape
        code = la.LA_BF16 if q.dtype == torch.bfloat16 else la.LA_F32
        nbytes = la.workspace_bytes("bwd", B, H, t["k"].shape[1], N, D, code, causal,
                                    t["cos_weight"] is not None, seg_len)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    out = la.fwd(t["q"], t["k"], t["v"], is_causal=causal, phi=phi, eps=eps,
                 cos_weight=t["cos_weight"], sin_weight=t["sin_weight"], seg_len=seg_len,
                 workspace=ws)
    grads = None
    if backward:
        grads = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], is_causal=causal, phi=phi, eps=eps,
                       cos_weight=t["cos_weight"], sin_weight=t["sin_weight"], seg_len=seg_len,
                       workspace=ws, state_from_fwd=saved)
    import torch
    torch.cuda.synchronize()
    return out, grads


def oracle_on(t, causal, phi, eps=1e-6, backward=True, groups=None):
    """Oracle outputs on the exact input values; ``groups`` = list of (b, g)
    pairs to restrict to (their n_rep query heads and KV head), else all."""
    q, k, v = np64(t["q"]), np64(t["k"]), np64(t["v"])
    g = np64(t.get("grad_out")) if backward else None
    cw, sw = np64(t["cos_weight"]), np64(t["sin_weight"])
    if groups is not None:
        parts = [oracle.group_slice(q, k, v, g, b, gg) for b, gg in groups]
        q = np.concatenate([p[0] for p in parts])
        k = np.concatenate([p[1] for p in parts])
        v = np.concatenate([p[2] for p in parts])
        g = np.concatenate([p[3] for p in parts]) if backward else None
    kw = dict(is_causal=causal, phi=phi, eps=eps, cos_weight=cw, sin_weight=sw)
    out = oracle.fwd(q, k, v, **kw)
    grads = oracle.bwd(q, k, v, g, **kw) if backward else None
    return out, grads


def select(x, groups, H, Hkv, kv=False):
    """Rows of a full [B, heads, N, D] GPU result matching oracle_on(groups)."""
    x = np64(x)
    if groups is None:
        return x
    nrep = H // Hkv
    if kv:
        return np.concatenate([x[b:b + 1, g:g + 1] for b, g in groups])
    return np.concatenate([x[b:b + 1, g * nrep:(g + 1) * nrep] for b, g in groups])


def compare(t, gpu_out, gpu_grads, ref_out, ref_grads, dtype, H, Hkv, groups=None, label="",
            blocks=True, grad_blocks=True):
    """Gate every output tensor whole and (blocks=True) per block of BLOCK
    rows, at the storage type's tolerance; grad_blocks=False leaves dq and dk
    to the whole-tensor gate (cases whose gradients are, by construction,
    small differences of large terms: one row with eps comparable to the
    weights)."""
    tol = TOL[dtype]
    pairs = {"out": (select(gpu_out, groups, H, Hkv), ref_out)}
    if gpu_grads is not None:
        dq, dk, dv = gpu_grads
        pairs["dq"] = (select(dq, groups, H, Hkv), ref_grads[0])
        pairs["dk"] = (select(dk, groups, H, Hkv, kv=True), ref_grads[1])
        pairs["dv"] = (select(dv, groups, H, Hkv, kv=True), ref_grads[2])
    errs = {n: rel(a, b) for n, (a, b) in pairs.items()}
    berrs = {n: block_rel(a, b) for n, (a, b) in pairs.items()} if blocks else {}
    say("  %s errors %s, worst block %s (tol %g)" % (
        label, {k: "%.2e" % e for k, e in errs.items()}, {k: "%.2e" % e for k, e in berrs.items()}, tol))
    log = os.environ.get("PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"label": label, "dtype": dtype, "tol": tol, "whole": errs,
                                "worst_block": berrs, "block": BLOCK}) + "\n")
    for name, e in errs.items():
        assert np.isfinite(e) and e <= tol, (label, name, e, tol)
    for name, e in berrs.items():
        if not grad_blocks and name in ("dq", "dk"):
            continue
        assert np.isfinite(e) and e <= tol, (label, name, "per block", e, tol)
    return errs
