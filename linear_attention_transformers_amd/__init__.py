"""Fused feature-map linear attention for AMD MI355X (gfx950).

``fwd`` / ``bwd`` call the hand-written HIP kernels of ``liblinattn.so``
through its C ABI (``include/linattn.h``); see ``_binding`` for the argument
rules.  ``linear_attention`` is the torch.autograd form (``autograd``); ``gqa``
materialises grouped-query head expansion and its adjoint; ``lowrank`` is the
low-rank projection y = (x V^T) U^T + bias and its gradients.  Build
the library with ``python -m linear_attention_transformers_amd.build``.
"""
from ._binding import (LA_BF16, LA_ERR_HIP, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_F32,
                       LA_OK, LA_OP_BWD, LA_OP_FWD, LIB_PATH, PHI, LinearAttnError, bwd, fwd,
                       header_functions, is_supported, load_library, timing_collect,
                       timing_enable, workspace_bytes)
from .autograd import LinearAttention, linear_attention
from . import gqa, lowrank

__all__ = ["fwd", "bwd", "linear_attention", "gqa", "lowrank", "LinearAttention", "is_supported", "workspace_bytes", "load_library", "header_functions", "timing_enable", "timing_collect",
           "LinearAttnError", "LIB_PATH", "PHI", "LA_OK", "LA_ERR_INVALID", "LA_ERR_UNSUPPORTED",
           "LA_ERR_HIP", "LA_F32", "LA_BF16", "LA_OP_FWD", "LA_OP_BWD"]
