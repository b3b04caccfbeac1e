"""Materialised grouped-query head expansion and its adjoint on the GPU.

Same calls as the gqa page of the SVD_linear_Attention API ("Module
neuralops.core.triton_kernels.gqa": ``fwd``, ``bwd``, ``is_supported``).
``fwd`` repeats each of the ``num_kv_heads`` heads of k and v ``n_rep =
num_heads // num_kv_heads`` times in place (head h of the result is KV head
h // n_rep); ``bwd`` sums each group of n_rep expanded gradients back onto its
KV head.  Both run in liblinattn.so (``la_gqa_expand`` / ``la_gqa_reduce`` of
include/la_gqa.h); the attention entry points never need them, since they map
heads by index.  As on the page, equal head counts return the inputs.
"""
from __future__ import annotations

from ._binding import _check, _dtype_code, _ptr, _stream, load_library


def _check_pair(a, b, heads: int, name: str):
    import torch

    for nm, t in ((name + "[0]", a), (name + "[1]", b)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % nm)
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("%s must be a contiguous 4-D GPU tensor [B, heads, N, D]" % nm)
    if a.shape != b.shape or a.dtype != b.dtype or a.device != b.device:
        raise ValueError("the two tensors must share shape, dtype and device")
    if a.shape[1] != heads:
        raise ValueError("expected %d heads, got %d" % (heads, a.shape[1]))


def is_supported(k, v, num_kv_heads: int, num_heads: int, **kwargs) -> bool:
    """Whether fwd/bwd run on the GPU kernels for these arguments."""
    import torch

    try:
        load_library()
    except ImportError:
        return False
    if num_kv_heads <= 0 or num_heads <= 0 or num_heads % num_kv_heads != 0:
        return False
    return all(isinstance(t, torch.Tensor) and t.is_cuda and t.dim() == 4
               and t.dtype in (torch.float32, torch.bfloat16) for t in (k, v))


def fwd(k, v, num_kv_heads: int, num_heads: int, **kwargs):
    """(k_expanded, v_expanded), each [B, num_heads, N, D]."""
    import torch

    if num_kv_heads == num_heads:
        return k, v
    if num_kv_heads <= 0 or num_heads <= 0 or num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a positive multiple of num_kv_heads")
    lib = load_library()
    _check_pair(k, v, num_kv_heads, "(k, v)")
    B, _, N, D = k.shape
    ko = torch.empty((B, num_heads, N, D), dtype=k.dtype, device=k.device)
    vo = torch.empty_like(ko)
    st = lib.la_gqa_expand(_ptr(k), _ptr(v), _ptr(ko), _ptr(vo), B, num_kv_heads, num_heads, N, D,
                           _dtype_code(k), _stream(k.device))
    _check(lib, st)
    return ko, vo


def bwd(grad_k, grad_v, num_kv_heads: int, num_heads: int, **kwargs):
    """(grad_k, grad_v) summed over each KV head's n_rep expanded heads: [B, num_kv_heads, N, D]."""
    import torch

    if num_kv_heads == num_heads:
        return grad_k, grad_v
    if num_kv_heads <= 0 or num_heads <= 0 or num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a positive multiple of num_kv_heads")
    lib = load_library()
    _check_pair(grad_k, grad_v, num_heads, "(grad_k, grad_v)")
    B, _, N, D = grad_k.shape
    gk = torch.empty((B, num_kv_heads, N, D), dtype=grad_k.dtype, device=grad_k.device)
    gv = torch.empty_like(gk)
    st = lib.la_gqa_reduce(_ptr(grad_k), _ptr(grad_v), _ptr(gk), _ptr(gv), B, num_kv_heads,
                           num_heads, N, D, _dtype_code(grad_k), _stream(grad_k.device))
    _check(lib, st)
    return gk, gv
