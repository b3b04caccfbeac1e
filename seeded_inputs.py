"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws Gaussian inputs,
rounds them to the storage dtype and tabulates the per-position cos/sin
weights.  Both the GPU path (through its Python binding) and the CPU oracle
consume exactly the arrays produced here.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal`` in
float32, drawn in the order q [B,H,N,D], k [B,H_kv,N,D], v [B,H_kv,N,D],
grad_out [B,H,N,D]; q, k and v are multiplied by ``scale`` in float32; bf16
tensors are the round-to-nearest-even image of those float32 draws.  The
cos/sin weights are cos(pi*i/(2N)) and sin(pi*i/(2N)), i = 0..N-1, computed
in float64 and rounded once to float32.  The materialised GQA op draws its own
k, v, grad_k, grad_v (``gqa_draw``), the low-rank projection its x, U, V,
bias, grad_out (``lowrank_draw``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    D: int
    dtypes: tuple
    modes: tuple            # subset of ("causal", "bidir")
    phi: str
    scale: float            # multiplies q, k, v draws
    cos: bool = False
    backward: bool = True
    eps: float = 1e-6
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.N


# The five workloads the path is specified on (sizes as stated for the method's
# headline runs); names say what each one is.
WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", 1, 2, 2, 256, 32, ("f32",), ("bidir", "causal"), "elu+1", 1.0,
        note="tiny fp32 correctness case, both modes, fwd+bwd"),
    "causal_fwd_b4h16n4096d64": Workload(
        "causal_fwd_b4h16n4096d64", 4, 16, 16, 4096, 64, ("bf16",), ("causal",), "elu+1", 0.5,
        backward=False, note="causal forward only"),
    "bidir_enc_b16h12n2048d64": Workload(
        "bidir_enc_b16h12n2048d64", 16, 12, 12, 2048, 64, ("bf16", "f32"), ("bidir",), "relu",
        1.0, note="bidirectional encoder fwd+bwd"),
    "causal_train_b2h32n16384d128": Workload(
        "causal_train_b2h32n16384d128", 2, 32, 32, 16384, 128, ("bf16",), ("causal",), "elu+1",
        0.5, note="causal training step fwd+bwd (headline)"),
    "causal_gqa_cos_b1h32kv8n65536d128": Workload(
        "causal_gqa_cos_b1h32kv8n65536d128", 1, 32, 8, 65536, 128, ("bf16",), ("causal",),
        "relu", 0.5, cos=True, note="long causal GQA n_rep=4 with cos/sin weighting"),
}

HEADLINE = "causal_train_b2h32n16384d128"


def draw(B, H, Hkv, N, D, scale=1.0, seed=0, grad=True):
    """float32 NumPy draws: dict with q, k, v and (if grad) grad_out."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    out = {}
    s = np.float32(scale)
    if scale != 1.0:
        q *= s
        k *= s
        v *= s
    out["q"], out["k"], out["v"] = q, k, v
    if grad:
        out["grad_out"] = rng.standard_normal((B, H, N, D), dtype=np.float32)
    return out


def gqa_draw(B, H, Hkv, N, D, seed=0):
    """float32 draws for the materialised GQA expansion and its adjoint: k, v
    [B,H_kv,N,D] ~ 0.5 N(0,1) and grad_k, grad_v [B,H,N,D] ~ N(0,1), drawn in
    that order from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, N, D), dtype=np.float32) * np.float32(0.5)
    v = rng.standard_normal((B, Hkv, N, D), dtype=np.float32) * np.float32(0.5)
    gk = rng.standard_normal((B, H, N, D), dtype=np.float32)
    gv = rng.standard_normal((B, H, N, D), dtype=np.float32)
    return {"k": k, "v": v, "grad_k": gk, "grad_v": gv}


# The materialised GQA op, measured on the long GQA workload's head shapes.
GQA_OPS = {
    "gqa_expand_reduce_b1h32kv8n65536d128": dict(B=1, H=32, Hkv=8, N=65536, D=128, dtype="bf16"),
}


def lowrank_draw(M, n_in, rank, n_out, seed=0, lead=None):
    """float32 draws for the low-rank projection, in this order from
    ``default_rng(seed)``: x [*lead or M, n_in] ~ N(0,1), V [rank, n_in] ~
    N(0, 1/n_in), U [n_out, rank] ~ N(0, 1/rank), bias [n_out] ~ N(0,1)/10,
    grad_out [*lead or M, n_out] ~ N(0,1) (factor scales keep y of order 1)."""
    rng = np.random.default_rng(seed)
    shape = tuple(lead) if lead else (M,)
    x = rng.standard_normal((*shape, n_in), dtype=np.float32)
    V = rng.standard_normal((rank, n_in), dtype=np.float32) * np.float32(1.0 / math.sqrt(n_in))
    U = rng.standard_normal((n_out, rank), dtype=np.float32) * np.float32(1.0 / math.sqrt(rank))
    bias = rng.standard_normal(n_out, dtype=np.float32) * np.float32(0.1)
    g = rng.standard_normal((*shape, n_out), dtype=np.float32)
    return {"x": x, "V": V, "U": U, "bias": bias, "grad_out": g}


# The low-rank projection, measured at the headline workload's token count
# (B*N = 2*16384) and width (H*D = 32*128) with a quarter rank.
LOWRANK_OPS = {
    "lowrank_m32768_in4096_r1024_out4096": dict(M=32768, n_in=4096, rank=1024, n_out=4096),
}


def cos_sin(N):
    """float32 cos(pi*i/(2N)), sin(pi*i/(2N)) for i = 0..N-1."""
    i = np.arange(N, dtype=np.float64)
    ang = math.pi * i / (2.0 * N)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def to_torch(arrays, dtype, device="cpu"):
    """Convert float32 NumPy draws to torch tensors of ``dtype`` ('f32'/'bf16')."""
    import torch

    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    return {name: torch.from_numpy(a).to(device=device).to(tdt).contiguous()
            for name, a in arrays.items()}


def exact_f64(t):
    """Exact float64 NumPy image of a float32/bf16 torch tensor (any device)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def workload_inputs(w: Workload, dtype, device="cpu", seed=0):
    """Torch inputs of workload ``w`` in ``dtype`` plus float32 cos/sin (or None)."""
    import torch

    arrays = draw(w.B, w.H, w.Hkv, w.N, w.D, w.scale, seed, grad=w.backward)
    t = to_torch(arrays, dtype, device)
    if w.cos:
        c, s = cos_sin(w.N)
        t["cos_weight"] = torch.from_numpy(c).to(device)
        t["sin_weight"] = torch.from_numpy(s).to(device)
    else:
        t["cos_weight"] = t["sin_weight"] = None
    return t
