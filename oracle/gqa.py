"""Oracle of the materialised GQA head expansion and its adjoint -- TEST
INFRASTRUCTURE ONLY (tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may use it; the GPU library never does).

Follows the gqa page of the SVD_linear_Attention API ("Module
neuralops.core.triton_kernels.gqa"):

* ``expand`` (page function fwd): the result's head axis is the page's view
  (num_kv_heads, n_rep) with n_rep fastest, so KV head g fills result heads
  g*n_rep .. g*n_rep + n_rep - 1.
* ``reduce`` (page function bwd): the gradients viewed the same way, summed
  over the n_rep axis.

Arithmetic is float64 on exact float64 images of the inputs; ``round_to``
rounds once to the storage type (nearest, ties to even), written from the
definition of the format.  Pinned by ``tests/test_oracle_gqa.py`` (hand-worked
values, the adjoint identity, the library repeat, the linear-attention
oracle's own GQA mapping, rounding ties).
"""
from __future__ import annotations

import numpy as np


def expand(x, n_rep: int):
    """[B, H_kv, N, D] -> [B, H_kv * n_rep, N, D]: slot g*n_rep + r holds head g."""
    x = np.asarray(x, dtype=np.float64)
    B, Hkv, N, D = x.shape
    out = np.empty((B, Hkv * n_rep, N, D), dtype=np.float64)
    for g in range(Hkv):
        for r in range(n_rep):
            out[:, g * n_rep + r] = x[:, g]
    return out


def reduce(y, n_rep: int):
    """[B, H, N, D] -> [B, H / n_rep, N, D]: head g sums slots g*n_rep .. g*n_rep + n_rep - 1."""
    y = np.asarray(y, dtype=np.float64)
    B, H, N, D = y.shape
    if H % n_rep:
        raise ValueError("H must be a multiple of n_rep")
    Hkv = H // n_rep
    out = np.zeros((B, Hkv, N, D), dtype=np.float64)
    for g in range(Hkv):
        for r in range(n_rep):
            out[:, g] += y[:, g * n_rep + r]
    return out


def round_to(x, dtype: str):
    """Round float64 values once to 'f32' or 'bf16' (nearest, ties to even);
    returns their exact float64 images.

    bf16 keeps 8 significant bits and float32's exponent range: a normal value
    m * 2^e (1/2 <= |m| < 1) becomes rint(m * 2^8) * 2^(e - 8); below 2^-126
    the spacing is fixed at 2^-133.  np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) >= 2.0 ** 128):
        raise ValueError("values outside the finite bf16 range")
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    return np.where(np.abs(x) < 2.0 ** -126, sub, normal)
