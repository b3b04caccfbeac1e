"""ctypes binding of liblinattn.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI of
``include/linattn.h``; this module checks tensors, allocates outputs and the
workspace with ``torch.empty`` on the inputs' device, and passes raw device
pointers plus the current HIP stream.  There is no other implementation to
fall back to: if the library is missing, every call raises.

Python names and defaults follow the SVD_linear_Attention page "Module
neuralops.core.triton_kernels.linear_attn" (functions fwd, bwd, is_supported:
is_causal=False, phi='elu+1', eps=1e-6, cos_weight=None, sin_weight=None).
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblinattn.so")
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "linattn.h")

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_F32, LA_BF16 = 0, 1
LA_OP_FWD, LA_OP_BWD = 0, 1
PHI = {"elu+1": 0, "relu": 1, "identity": 2}
SUPPORTED_D = (32, 64, 128)

_lock = threading.Lock()
_lib = None


class KernelTime(ctypes.Structure):
    """Mirror of la_kernel_time."""
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int),
                ("total_ms", ctypes.c_double)]


def timing_enable(on: bool = True):
    """Bracket every later kernel launch of this thread with HIP events."""
    load_library().la_timing_enable(int(bool(on)))


def timing_collect(max_entries: int = 64):
    """{kernel name: (launches, total_ms)} of the launches recorded since the
    last collect (waits for them to finish)."""
    lib = load_library()
    buf = (KernelTime * max_entries)()
    n = lib.la_timing_collect(buf, max_entries)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}


class LinearAttnError(RuntimeError):
    """A non-OK status from the C library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load liblinattn.so and declare the prototypes of include/linattn.h."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise ImportError(
                "liblinattn.so is not built (%s); run "
                "`python -m linear_attention_transformers_amd.build`" % path)
        lib = ctypes.CDLL(path)
        vp, sz, i, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
        fp = ctypes.POINTER(ctypes.c_float)
        lib.la_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
        lib.la_workspace_bytes.restype = sz
        lib.la_workspace_bytes_ex.argtypes = [i, i, i, i, i, i, i, i, i, i]
        lib.la_workspace_bytes_ex.restype = sz
        fwd_args = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, fp, fp, vp, sz, vp]
        bwd_args = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, fp, fp, vp, sz, vp]
        lib.la_fwd.argtypes = fwd_args
        lib.la_fwd_ex.argtypes = fwd_args + [i]
        lib.la_fwd_noalloc.argtypes = fwd_args[:15] + [vp]
        lib.la_fwd_noalloc.restype = i
        lib.la_bwd.argtypes = bwd_args
        lib.la_bwd_ex.argtypes = bwd_args + [i]
        lib.la_bwd_saved.argtypes = bwd_args
        lib.la_bwd_saved_ex.argtypes = bwd_args + [i]
        for fn in (lib.la_fwd, lib.la_fwd_ex, lib.la_bwd, lib.la_bwd_ex, lib.la_bwd_saved,
                   lib.la_bwd_saved_ex):
            fn.restype = i
        lib.la_status_string.argtypes = [i]
        lib.la_status_string.restype = ctypes.c_char_p
        lib.la_last_error.argtypes = []
        lib.la_last_error.restype = ctypes.c_char_p
        lib.la_timing_enable.argtypes = [i]
        lib.la_timing_enable.restype = i
        lib.la_timing_collect.argtypes = [ctypes.POINTER(KernelTime), i]
        lib.la_timing_collect.restype = i
        gqa_args = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
        lib.la_gqa_expand.argtypes = gqa_args
        lib.la_gqa_reduce.argtypes = gqa_args
        lib.la_gqa_expand.restype = i
        lib.la_gqa_reduce.restype = i
        lib.la_lowrank_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.la_lowrank_workspace_bytes.restype = sz
        lib.la_lowrank_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        lib.la_lowrank_fwd.restype = i
        lib.la_lowrank_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        lib.la_lowrank_bwd.restype = i
        if path == LIB_PATH:
            _lib = lib
        return lib


def header_functions(header: str | None = None):
    """Names of the functions a header declares (default: every include/*.h)."""
    paths = [header] if header else sorted(
        os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
    names = set()
    for path in paths:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def _check(lib, st: int):
    if st != LA_OK:
        msg = lib.la_last_error().decode() or lib.la_status_string(st).decode()
        if st in (LA_ERR_INVALID, LA_ERR_UNSUPPORTED):
            raise ValueError("%s: %s" % (lib.la_status_string(st).decode(), msg))
        raise LinearAttnError(st, msg)


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise ValueError("tensors must be float32 or bfloat16, got %s" % (t.dtype,))


def _validate(q, k, v, cos_weight, sin_weight, grad_out=None):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("grad_out", grad_out)):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.dim() != 4:
            raise ValueError("%s must be 4-D [B, heads, N, D]" % name)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.dtype != k.dtype or q.dtype != v.dtype or (grad_out is not None and grad_out.dtype != q.dtype):
        raise ValueError("q, k, v (and grad_out) must share one dtype")
    B, H, N, D = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k/v must be [B, H_kv, N, D] matching q's B, N, D")
    if grad_out is not None and grad_out.shape != q.shape:
        raise ValueError("grad_out must have q's shape")
    dev = q.device
    for t in (k, v, grad_out):
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on one device")
    if (cos_weight is None) != (sin_weight is None):
        raise ValueError("cos_weight and sin_weight must be given together")
    if cos_weight is not None:
        for name, t in (("cos_weight", cos_weight), ("sin_weight", sin_weight)):
            if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != N or t.device != dev:
                raise ValueError("%s must be a contiguous float32 [N] tensor on q's device" % name)
    return B, H, k.shape[1], N, D


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _fptr(t):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float)) \
        if t is not None else None


def _stream(dev):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_bytes(op: str, B, H, H_kv, N, D, dtype_code, causal, has_cos, seg_len=0) -> int:
    lib = load_library()
    return int(lib.la_workspace_bytes_ex(LA_OP_FWD if op == "fwd" else LA_OP_BWD, B, H, H_kv,
                                         N, D, dtype_code, int(bool(causal)),
                                         int(bool(has_cos)), int(seg_len)))


def is_supported(q, k, v, **kwargs) -> bool:
    """Whether fwd/bwd serve these tensors (GPU, float32/bfloat16, D in 32/64/128)."""
    import torch

    try:
        load_library()
    except ImportError:
        return False
    return (isinstance(q, torch.Tensor) and q.is_cuda and q.dim() == 4
            and q.dtype in (torch.float32, torch.bfloat16) and q.shape[-1] in SUPPORTED_D)


def fwd(q, k, v, is_causal: bool = False, phi: str = "elu+1", eps: float = 1e-6,
        cos_weight=None, sin_weight=None, seg_len: int = 0, out=None, workspace=None):
    """Forward: out [B,H,N,D] from q [B,H,N,D], k, v [B,H_kv,N,D]."""
    import torch

    lib = load_library()
    B, H, Hkv, N, D = _validate(q, k, v, cos_weight, sin_weight)
    if phi not in PHI:
        raise ValueError("phi must be one of %s" % sorted(PHI))
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    nbytes = workspace_bytes("fwd", B, H, Hkv, N, D, code, is_causal, cos_weight is not None,
                             seg_len)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.la_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, D, code,
                       int(bool(is_causal)), PHI[phi], float(eps), _fptr(cos_weight),
                       _fptr(sin_weight), _ptr(workspace), workspace.numel(), _stream(q.device),
                       int(seg_len))
    _check(lib, st)
    return out


def bwd(q, k, v, grad_out, is_causal: bool = False, phi: str = "elu+1", eps: float = 1e-6,
        cos_weight=None, sin_weight=None, seg_len: int = 0, workspace=None, grads=None,
        state_from_fwd: bool = False):
    """Backward: (dq [B,H,N,D], dk [B,H_kv,N,D], dv [B,H_kv,N,D]) of fwd for grad_out.

    state_from_fwd: `workspace` is the one the forward on these same inputs and
    arguments was given (sized by workspace_bytes("bwd", ...)) and still holds
    its state records, which the backward then reuses (la_bwd_saved)."""
    import torch

    lib = load_library()
    B, H, Hkv, N, D = _validate(q, k, v, cos_weight, sin_weight, grad_out)
    if phi not in PHI:
        raise ValueError("phi must be one of %s" % sorted(PHI))
    code = _dtype_code(q)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() \
                    or t.device != ref.device:
                raise ValueError("%s must be a contiguous tensor like %s" % (name, "q" if name == "dq" else "k"))
    nbytes = workspace_bytes("bwd", B, H, Hkv, N, D, code, is_causal, cos_weight is not None,
                             seg_len)
    if state_from_fwd:
        if workspace is None or workspace.numel() < nbytes:
            raise ValueError("state_from_fwd needs the forward's workspace, of at least %d bytes"
                             % nbytes)
    elif workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    entry = lib.la_bwd_saved_ex if state_from_fwd else lib.la_bwd_ex
    st = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(grad_out), _ptr(dq), _ptr(dk), _ptr(dv),
                       B, H, Hkv, N, D, code, int(bool(is_causal)), PHI[phi], float(eps),
                       _fptr(cos_weight), _fptr(sin_weight), _ptr(workspace), workspace.numel(),
                       _stream(q.device), int(seg_len))
    _check(lib, st)
    return dq, dk, dv
