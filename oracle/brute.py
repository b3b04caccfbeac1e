"""O(N^2) brute force of feature-map linear attention -- TEST INFRASTRUCTURE ONLY.

The kernelised-attention sum written out directly, one head at a time:

    W = (Phi(Q) Phi(K)^T) * M,   out = W V / (W 1 + eps)

with M the lower-triangular mask (diagonal included) for causal runs and all
ones otherwise; Phi is phi, or [cos*phi, sin*phi] when cos/sin weights are
given (linear_attn page, module docstring and fwd arguments).  Query head h
uses KV head h // n_rep (gqa page, bwd: the head axis viewed as
(H_kv, n_rep)).  It shares no code with the C oracle; the tests pin one against
the other.  ``torch_out`` is the same sum in float64 PyTorch ops so that
``torch.autograd`` (the routine the linear_attn page's bwd calls) gives the
reference gradient.
"""
from __future__ import annotations

import numpy as np


def phi_np(x, phi):
    if phi == "elu+1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    if phi == "relu":
        return np.maximum(x, 0.0)
    if phi == "identity":
        return x
    raise ValueError(phi)


def features_np(x, phi, cos_weight=None, sin_weight=None):
    """x [..., N, D] -> Phi(x) [..., N, F]."""
    f = phi_np(np.asarray(x, np.float64), phi)
    if cos_weight is None:
        return f
    cw = np.asarray(cos_weight, np.float64)[:, None]
    sw = np.asarray(sin_weight, np.float64)[:, None]
    return np.concatenate([cw * f, sw * f], axis=-1)


def weights_np(q, k, is_causal, phi, cos_weight=None, sin_weight=None):
    """W [B,H,N,N] with query head h paired with KV head h // n_rep."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    H, Hkv = q.shape[1], k.shape[1]
    kv_of = np.arange(H) // (H // Hkv)
    qf = features_np(q, phi, cos_weight, sin_weight)
    kf = features_np(k, phi, cos_weight, sin_weight)[:, kv_of]
    W = qf @ np.swapaxes(kf, -1, -2)
    if is_causal:
        N = q.shape[2]
        W = W * np.tril(np.ones((N, N)))
    return W


def out_np(q, k, v, is_causal=False, phi="elu+1", eps=1e-6, cos_weight=None, sin_weight=None):
    v = np.asarray(v, np.float64)
    H, Hkv = q.shape[1], v.shape[1]
    kv_of = np.arange(H) // (H // Hkv)
    W = weights_np(q, k, is_causal, phi, cos_weight, sin_weight)
    return (W @ v[:, kv_of]) / (W.sum(-1, keepdims=True) + eps)


def torch_out(q, k, v, is_causal=False, phi="elu+1", eps=1e-6, cos_weight=None,
              sin_weight=None):
    """Same sum on float64 torch tensors (differentiable in q, k, v)."""
    import torch

    def phi_t(x):
        if phi == "elu+1":
            return torch.nn.functional.elu(x) + 1.0
        if phi == "relu":
            return torch.relu(x)
        return x

    def feats(x):
        f = phi_t(x)
        if cos_weight is None:
            return f
        cw = torch.as_tensor(np.asarray(cos_weight, np.float64))[:, None]
        sw = torch.as_tensor(np.asarray(sin_weight, np.float64))[:, None]
        return torch.cat([cw * f, sw * f], dim=-1)

    H, Hkv = q.shape[1], k.shape[1]
    kv_of = torch.arange(H) // (H // Hkv)
    qf = feats(q)
    kf = feats(k)[:, kv_of]
    W = qf @ kf.transpose(-1, -2).contiguous()
    if is_causal:
        N = q.shape[2]
        W = W * torch.tril(torch.ones(N, N, dtype=W.dtype))
    return (W @ v[:, kv_of]) / (W.sum(-1, keepdim=True) + eps)


def torch_grads(q, k, v, grad_out, **kw):
    """(dq, dk, dv) by torch.autograd through ``torch_out`` in float64."""
    import torch

    qt = torch.tensor(np.asarray(q, np.float64), requires_grad=True)
    kt = torch.tensor(np.asarray(k, np.float64), requires_grad=True)
    vt = torch.tensor(np.asarray(v, np.float64), requires_grad=True)
    out = torch_out(qt, kt, vt, **kw)
    gq, gk, gv = torch.autograd.grad(out, [qt, kt, vt],
                                     torch.tensor(np.asarray(grad_out, np.float64)))
    return gq.numpy(), gk.numpy(), gv.numpy()
