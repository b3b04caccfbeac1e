"""Oracle of the low-rank projection, forward and backward -- TEST
INFRASTRUCTURE ONLY (tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may use it; the GPU library never does).

Follows the low_rank page of the SVD_linear_Attention API ("Module
neuralops.core.triton_kernels.low_rank"): ``fwd`` computes
y = (x V^T) U^T + bias for x [..., in], V [rank, in], U [out, rank] and an
optional bias [out]; ``bwd`` returns the gradients of that expression with
respect to x, U, V and bias for a given grad_out (the page obtains them by
autograd).  Written out with t = x V^T and g = grad_out, flattening x's
leading axes into M rows:

    grad_t    = g U                      [M, rank]
    grad_x    = grad_t V                 [M, in]
    grad_U    = g^T t                    [out, rank]
    grad_V    = grad_t^T x               [rank, in]
    grad_bias = sum over rows of g       [out]

Float64 throughout on exact float64 images of the inputs; NumPy matmul is the
only primitive.  Pinned by ``tests/test_oracle_lowrank.py`` (a hand-worked
example, finite differences, the identity projection, the other association
order, and planted mistakes).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def fwd(x, U, V, bias=None):
    """y [..., out] = (x V^T) U^T + bias."""
    x, U, V = _f64(x), _f64(U), _f64(V)
    t = x @ V.T
    y = t @ U.T
    if bias is not None:
        y = y + _f64(bias)
    return y


def bwd(x, U, V, grad_out, bias=None):
    """(grad_x, grad_U, grad_V, grad_bias or None) of fwd at (x, U, V, bias) for grad_out."""
    x, U, V, g = _f64(x), _f64(U), _f64(V), _f64(grad_out)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    g2 = g.reshape(-1, g.shape[-1])
    t = x2 @ V.T
    grad_t = g2 @ U
    grad_x = (grad_t @ V).reshape(*lead, V.shape[1])
    grad_U = g2.T @ t
    grad_V = grad_t.T @ x2
    grad_b = g2.sum(axis=0) if bias is not None else None
    return grad_x, grad_U, grad_V, grad_b
