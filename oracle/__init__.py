"""CPU oracle for fused feature-map linear attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it: the two share no code.

Contents
--------
* ``linattn_oracle.c`` -- the fp64 token-recurrent definition (forward and
  backward) plus its chunk form, loaded here through ctypes.
* ``brute``            -- an O(N^2) NumPy brute force and a float64 PyTorch
  autograd gradient of it, for tiny inputs.

Every function takes NumPy arrays (any float dtype; upcast exactly to float64)
in the layout q/grad_out [B,H,N,D], k/v [B,H_kv,N,D], cos/sin [N], and returns
float64 arrays.  Parity is pinned for every function here by the CPU tests in
``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LOCK = threading.Lock()
_LIB = None

PHI = {"elu+1": 0, "relu": 1, "identity": 2}


def build(force: bool = True, src: str = _SRC, out: str = _SO) -> str:
    """Compile the C oracle with gcc (OpenMP); ``src``/``out`` default to the
    committed source and the library next to it."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Werror",
             "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(q, k, v, phi, cos_weight, sin_weight):
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,H,N,D] and k, v [B,H_kv,N,D]")
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("q and k/v disagree on B, N or D")
    if (cos_weight is None) != (sin_weight is None):
        raise ValueError("cos_weight and sin_weight go together")
    cw = sw = None
    if cos_weight is not None:
        cw, sw = _f64(cos_weight).reshape(-1), _f64(sin_weight).reshape(-1)
        if cw.shape[0] != N or sw.shape[0] != N:
            raise ValueError("cos/sin weights must have N entries")
    if phi not in PHI:
        raise ValueError("unknown feature map %r" % (phi,))
    return q, k, v, cw, sw, (B, H, Hkv, N, D)


class Oracle:
    """ctypes front end of one compiled copy of ``linattn_oracle.c``."""

    def __init__(self, so_path: str):
        lib = ctypes.CDLL(so_path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        d = ctypes.c_double
        lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d, dp, dp]
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d, dp, dp]
        lib.oracle_fwd_chunked.argtypes = [dp, dp, dp, dp, i, i, i, i, i, i, i, d, dp, dp, i]
        lib.oracle_bwd_chunked.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, i, d,
                                           dp, dp, i]
        for fn in (lib.oracle_fwd, lib.oracle_bwd, lib.oracle_fwd_chunked,
                   lib.oracle_bwd_chunked):
            fn.restype = ctypes.c_int
        self.lib = lib

    def fwd(self, q, k, v, is_causal=False, phi="elu+1", eps=1e-6, cos_weight=None,
            sin_weight=None, return_den=False):
        """Token-recurrent forward (the definition).  Returns out [B,H,N,D]
        (and den [B,H,N] = Phi(q_i).z_i + eps when ``return_den``)."""
        q, k, v, cw, sw, (B, H, Hkv, N, D) = _prep(q, k, v, phi, cos_weight, sin_weight)
        out = np.empty((B, H, N, D), np.float64)
        den = np.empty((B, H, N), np.float64)
        rc = self.lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(den), B, H, Hkv,
                                 N, D, int(bool(is_causal)), PHI[phi], float(eps), _ptr(cw),
                                 _ptr(sw))
        if rc:
            raise ValueError("oracle_fwd rejected its arguments (code %d)" % rc)
        return (out, den) if return_den else out

    def bwd(self, q, k, v, grad_out, is_causal=False, phi="elu+1", eps=1e-6,
            cos_weight=None, sin_weight=None):
        """Token-recurrent backward: (dq [B,H,N,D], dk [B,H_kv,N,D], dv [B,H_kv,N,D])."""
        q, k, v, cw, sw, (B, H, Hkv, N, D) = _prep(q, k, v, phi, cos_weight, sin_weight)
        g = _f64(grad_out)
        if g.shape != q.shape:
            raise ValueError("grad_out must match q")
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        rc = self.lib.oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, H, Hkv, N, D, int(bool(is_causal)), PHI[phi],
                                 float(eps), _ptr(cw), _ptr(sw))
        if rc:
            raise ValueError("oracle_bwd rejected its arguments (code %d)" % rc)
        return dq, dk, dv

    def fwd_chunked(self, q, k, v, chunk, is_causal=False, phi="elu+1", eps=1e-6,
                    cos_weight=None, sin_weight=None):
        """Chunk form of the forward with chunk length ``chunk``."""
        q, k, v, cw, sw, (B, H, Hkv, N, D) = _prep(q, k, v, phi, cos_weight, sin_weight)
        out = np.empty((B, H, N, D), np.float64)
        rc = self.lib.oracle_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N,
                                         D, int(bool(is_causal)), PHI[phi], float(eps),
                                         _ptr(cw), _ptr(sw), int(chunk))
        if rc:
            raise ValueError("oracle_fwd_chunked rejected its arguments (code %d)" % rc)
        return out

    def bwd_chunked(self, q, k, v, grad_out, chunk, is_causal=False, phi="elu+1", eps=1e-6,
                    cos_weight=None, sin_weight=None):
        """Chunk form of the backward with chunk length ``chunk``."""
        q, k, v, cw, sw, (B, H, Hkv, N, D) = _prep(q, k, v, phi, cos_weight, sin_weight)
        g = _f64(grad_out)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        rc = self.lib.oracle_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq),
                                         _ptr(dk), _ptr(dv), B, H, Hkv, N, D,
                                         int(bool(is_causal)), PHI[phi], float(eps), _ptr(cw),
                                         _ptr(sw), int(chunk))
        if rc:
            raise ValueError("oracle_bwd_chunked rejected its arguments (code %d)" % rc)
        return dq, dk, dv


def load(so_path: str = _SO) -> Oracle:
    return Oracle(so_path)


def _default() -> Oracle:
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(_SO):
                build(force=True)
            _LIB = Oracle(_SO)
    return _LIB


def fwd(*args, **kw):
    return _default().fwd(*args, **kw)


def bwd(*args, **kw):
    return _default().bwd(*args, **kw)


def fwd_chunked(*args, **kw):
    return _default().fwd_chunked(*args, **kw)


def bwd_chunked(*args, **kw):
    return _default().bwd_chunked(*args, **kw)


def group_slice(q, k, v, grad_out, b, g):
    """The sub-problem of one (batch, KV head) group: its n_rep query heads and
    their shared k, v, at full N.  The oracle on this slice equals the oracle
    on the whole problem restricted to those heads, because groups never
    interact."""
    H, Hkv = q.shape[1], k.shape[1]
    nrep = H // Hkv
    sl = slice(g * nrep, (g + 1) * nrep)
    out = [q[b:b + 1, sl], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1]]
    out.append(None if grad_out is None else grad_out[b:b + 1, sl])
    return out
