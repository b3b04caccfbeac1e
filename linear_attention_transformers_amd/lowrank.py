"""Low-rank projection y = (x V^T) U^T + bias on the GPU matrix cores.

Same calls as the low_rank page of the SVD_linear_Attention API ("Module
neuralops.core.triton_kernels.low_rank": ``fwd``, ``bwd``, ``is_supported``),
run by liblinattn.so (``la_lowrank_fwd`` / ``la_lowrank_bwd`` of
include/la_lowrank.h).  x may have any leading axes (flattened into rows);
U is [out, rank], V [rank, in], bias [out] or None; every tensor is bf16.
``LowRankProjection`` is the torch.autograd form.
"""
from __future__ import annotations

from ._binding import LA_BF16, LA_OP_BWD, LA_OP_FWD, _check, _ptr, _stream, load_library


def _check_args(x, U, V, bias, extra=()):
    import torch

    for name, t in (("x", x), ("U", U), ("V", V), ("bias", bias)) + tuple(extra):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16 or t.device != x.device:
            raise ValueError("%s must be a contiguous bfloat16 tensor on x's device" % name)
    if U.dim() != 2 or V.dim() != 2 or U.shape[1] != V.shape[0] or x.shape[-1] != V.shape[1]:
        raise ValueError("expected x [..., in], V [rank, in], U [out, rank]")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != U.shape[0]):
        raise ValueError("bias must be [out]")
    n_in, rank, n_out = V.shape[1], V.shape[0], U.shape[0]
    M = x.numel() // n_in
    return M, n_in, rank, n_out


def _workspace(op, M, n_in, rank, n_out, device, workspace):
    import torch

    lib = load_library()
    need = int(lib.la_lowrank_workspace_bytes(op, M, n_in, rank, n_out, LA_BF16))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace


def is_supported(x, U, V, bias=None, **kwargs) -> bool:
    """Whether fwd/bwd run on the GPU kernels: bf16 GPU tensors, in / rank / out multiples of 8."""
    import torch

    try:
        load_library()
    except ImportError:
        return False
    ts = [t for t in (x, U, V, bias) if t is not None]
    if not all(isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 for t in ts):
        return False
    if U.dim() != 2 or V.dim() != 2 or U.shape[1] != V.shape[0] or x.shape[-1] != V.shape[1]:
        return False
    return all(d >= 8 and d % 8 == 0 for d in (V.shape[1], V.shape[0], U.shape[0]))


def fwd(x, U, V, bias=None, workspace=None, **kwargs):
    """y [..., out] = (x V^T) U^T + bias."""
    import torch

    lib = load_library()
    M, n_in, rank, n_out = _check_args(x, U, V, bias)
    y = torch.empty((*x.shape[:-1], n_out), dtype=x.dtype, device=x.device)
    ws = _workspace(LA_OP_FWD, M, n_in, rank, n_out, x.device, workspace)
    st = lib.la_lowrank_fwd(_ptr(x), _ptr(U), _ptr(V), _ptr(bias), _ptr(y), M, n_in, rank, n_out, LA_BF16,
                            _ptr(ws), ws.numel(), _stream(x.device))
    _check(lib, st)
    return y


def bwd(x, U, V, grad_out, bias=None, workspace=None, **kwargs):
    """(grad_x, grad_U, grad_V, grad_bias or None) of fwd for grad_out."""
    import torch

    lib = load_library()
    M, n_in, rank, n_out = _check_args(x, U, V, bias, (("grad_out", grad_out),))
    if grad_out.shape != (*x.shape[:-1], n_out):
        raise ValueError("grad_out must be [..., out]")
    gx, gU, gV = torch.empty_like(x), torch.empty_like(U), torch.empty_like(V)
    gb = torch.empty_like(bias) if bias is not None else None
    ws = _workspace(LA_OP_BWD, M, n_in, rank, n_out, x.device, workspace)
    st = lib.la_lowrank_bwd(_ptr(x), _ptr(U), _ptr(V), _ptr(grad_out), _ptr(gx), _ptr(gU), _ptr(gV),
                            _ptr(gb), M, n_in, rank, n_out, LA_BF16, _ptr(ws), ws.numel(),
                            _stream(x.device))
    _check(lib, st)
    return gx, gU, gV, gb


def _autograd():
    import torch

    class LowRankProjection(torch.autograd.Function):
        """torch.autograd form: forward saves x, U, V, bias; backward is ``bwd``."""

        @staticmethod
        def forward(ctx, x, U, V, bias=None):
            ctx.save_for_backward(x, U, V, bias)
            return fwd(x, U, V, bias)

        @staticmethod
        def backward(ctx, grad_out):
            x, U, V, bias = ctx.saved_tensors
            gx, gU, gV, gb = bwd(x, U, V, grad_out.contiguous(), bias)
            return gx, gU, gV, gb

    return LowRankProjection


def low_rank_projection(x, U, V, bias=None):
    """y = (x V^T) U^T + bias with gradients through ``bwd``."""
    return _autograd().apply(x, U, V, bias)
