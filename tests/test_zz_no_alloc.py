"""la_fwd_noalloc -- the forward with its workspace in the library's static
device array, for callers that cannot allocate -- through the C ABI, against
la_fwd with a caller-allocated workspace: bitwise equal, on calls in a row
whose second is smaller than the first (the array keeps the previous call's
contents, which must not matter), and sizes beyond the array's limit are
rejected before anything is launched."""
import ctypes

import pytest

import seeded_inputs as si
from parity_util import gpu_or_skip, make, say

pytestmark = pytest.mark.gpu

LIMIT = 40 << 20   # LA_NOALLOC_SCRATCH_BYTES

# (B, H, H_kv, N, D, storage, causal, cos/sin, phi): the headline forward
# (36.3 MiB of state records), then smaller cases on other kernel families
CASES = [(2, 32, 32, 16384, 128, "bf16", True, False, "elu+1"),
         (1, 4, 2, 300, 64, "bf16", True, True, "relu"),
         (1, 2, 2, 256, 32, "f32", False, False, "elu+1")]


def _call(la, lib, t, B, H, Hkv, N, D, dtype, causal, phi, out, ws=None):
    import torch
    P = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    F = lambda x: ctypes.cast(ctypes.c_void_p(x.data_ptr()), ctypes.POINTER(ctypes.c_float)) \
        if x is not None else None
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (P(t["q"]), P(t["k"]), P(t["v"]), P(out), B, H, Hkv, N, D, code, int(causal),
            la.PHI[phi], ctypes.c_float(1e-6), F(t["cos_weight"]), F(t["sin_weight"]))
    if ws is None:
        return lib.la_fwd_noalloc(*args, stream)
    return lib.la_fwd(*args, P(ws), ws.numel(), stream)


def test_noalloc_equals_la_fwd_twice():
    torch, la = gpu_or_skip()
    lib = la.load_library()
    for case in CASES:
        B, H, Hkv, N, D, dtype, causal, cos, phi = case
        say("noalloc case %s" % (case,))
        t = make(B, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=N)
        code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
        need = la.workspace_bytes("fwd", B, H, Hkv, N, D, code, causal, cos)
        assert 0 < need <= LIMIT, need
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = torch.empty_like(t["q"])
        got = torch.full_like(t["q"], float("nan"))
        assert _call(la, lib, t, B, H, Hkv, N, D, dtype, causal, phi, ref, ws) == la.LA_OK
        st = _call(la, lib, t, B, H, Hkv, N, D, dtype, causal, phi, got)
        assert st == la.LA_OK, lib.la_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), case
        del t, ws, ref, got


def test_noalloc_rejects_sizes_beyond_the_limit():
    torch, la = gpu_or_skip()
    lib = la.load_library()
    B, H, Hkv, N, D = 4, 32, 32, 16384, 128   # 72.6 MiB of state records
    assert la.workspace_bytes("fwd", B, H, Hkv, N, D, la.LA_BF16, True, False) > LIMIT
    small = make(1, 1, 1, 64, 128, "bf16")   # pointers only: nothing may be launched
    out = torch.empty_like(small["q"])
    st = _call(la, lib, small, B, H, Hkv, N, D, "bf16", True, "elu+1", out)
    assert st == la.LA_ERR_INVALID
    assert "LA_NOALLOC_SCRATCH_BYTES" in lib.la_last_error().decode()
