"""torch.autograd integration of the library's forward and backward.

``linear_attention(q, k, v, ...)`` is differentiable in q, k and v.  Its
forward runs ``fwd`` with a workspace sized for the backward and keeps it,
with q, k and v, for the backward, which then reuses the forward's state
records instead of computing them again (``bwd(..., state_from_fwd=True)``,
C ABI ``la_bwd_saved``).  No gradient flows to cos_weight, sin_weight or eps:
the backward of the linear_attn page returns the three input gradients only.
The backward is not itself differentiable (no second derivatives).
"""
import torch
from torch.autograd.function import once_differentiable

from . import _binding


class LinearAttention(torch.autograd.Function):
    """Autograd function over fwd / bwd; see ``linear_attention``."""

    @staticmethod
    def forward(ctx, q, k, v, is_causal, phi, eps, cos_weight, sin_weight, seg_len):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        B, H, Hkv, N, D = _binding._validate(q, k, v, cos_weight, sin_weight)
        nbytes = _binding.workspace_bytes("bwd", B, H, Hkv, N, D, _binding._dtype_code(q),
                                          is_causal, cos_weight is not None, seg_len)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        out = _binding.fwd(q, k, v, is_causal, phi, eps, cos_weight, sin_weight,
                           seg_len=seg_len, workspace=ws)
        ctx.save_for_backward(q, k, v, cos_weight, sin_weight)
        ctx.ws = ws
        ctx.args = (is_causal, phi, eps, seg_len)
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_out):
        q, k, v, cos_weight, sin_weight = ctx.saved_tensors
        is_causal, phi, eps, seg_len = ctx.args
        dq, dk, dv = _binding.bwd(q, k, v, grad_out.contiguous(), is_causal, phi, eps,
                                  cos_weight, sin_weight, seg_len=seg_len, workspace=ctx.ws,
                                  state_from_fwd=True)
        return dq, dk, dv, None, None, None, None, None, None


def linear_attention(q, k, v, is_causal: bool = False, phi: str = "elu+1", eps: float = 1e-6,
                     cos_weight=None, sin_weight=None, seg_len: int = 0):
    """Differentiable fused linear attention: out [B,H,N,D] from q [B,H,N,D],
    k, v [B,H_kv,N,D] (arguments as ``fwd``)."""
    return LinearAttention.apply(q, k, v, bool(is_causal), phi, float(eps), cos_weight,
                                 sin_weight, int(seg_len))
