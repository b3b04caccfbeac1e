"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the CPU oracle on the same seeded inputs, compare normwise.

Tolerances (max |gpu - oracle| / max |oracle| per output tensor): 1e-4 for
float32 storage, 2e-2 for bfloat16 storage with float32 accumulation.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import seeded_inputs as si

TOL = {"f32": 1e-4, "bf16": 2e-2}


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


def run_gpu(la, t, causal, phi, eps=1e-6, seg_len=0, backward=True):
    out = la.fwd(t["q"], t["k"], t["v"], is_causal=causal, phi=phi, eps=eps,
                 cos_weight=t["cos_weight"], sin_weight=t["sin_weight"], seg_len=seg_len)
    grads = None
    if backward:
        grads = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], is_causal=causal, phi=phi, eps=eps,
                       cos_weight=t["cos_weight"], sin_weight=t["sin_weight"], seg_len=seg_len)
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


def compare(t, gpu_out, gpu_grads, ref_out, ref_grads, dtype, H, Hkv, groups=None, label=""):
    tol = TOL[dtype]
    errs = {"out": rel(select(gpu_out, groups, H, Hkv), ref_out)}
    if gpu_grads is not None:
        dq, dk, dv = gpu_grads
        errs["dq"] = rel(select(dq, groups, H, Hkv), ref_grads[0])
        errs["dk"] = rel(select(dk, groups, H, Hkv, kv=True), ref_grads[1])
        errs["dv"] = rel(select(dv, groups, H, Hkv, kv=True), ref_grads[2])
    say("  %s errors %s (tol %g)" % (label, {k: "%.2e" % e for k, e in errs.items()}, tol))
    for name, e in errs.items():
        assert np.isfinite(e) and e <= tol, (label, name, e, tol)
    return errs
