"""GPU parity of the materialised GQA expansion and its adjoint (la_gqa_expand /
la_gqa_reduce, through the C ABI and linear_attention_transformers_amd.gqa)
against oracle/gqa.py on the same seeded inputs.

The expansion is byte work and the sum is the exact float64 sum rounded once
to the storage type on both sides, so every comparison is bitwise.  Cases:
the 16-byte vector path with ragged block tails, the element path (slab size
not a multiple of 16 bytes, or a base off 16-byte alignment), k alone (v pair
NULL), n_rep = 1, 12 seeded random shapes, and the long GQA workload's shapes
at full size on sampled rows."""
import ctypes

import numpy as np
import pytest

import seeded_inputs as si
from oracle import gqa as og
from parity_util import gpu_or_skip, say

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1}


def _inputs(torch, B, Hkv, H, N, D, dtype, seed):
    t = si.to_torch(si.gqa_draw(B, H, Hkv, N, D, seed), dtype, "cuda")
    return t["k"], t["v"], t["grad_k"], t["grad_v"]


def _f64(t):
    return si.exact_f64(t)


CASES = []
for dtype in ("bf16", "f32"):
    for (B, Hkv, nrep, N, D) in [(2, 3, 2, 37, 64), (1, 2, 4, 300, 128), (3, 1, 8, 5, 32),
                                 (2, 2, 1, 17, 64), (1, 3, 3, 1, 8)]:
        CASES.append((dtype, B, Hkv, nrep, N, D))
    CASES.append((dtype, 2, 2, 4, 37, 3))    # element path: slab bytes not a multiple of 16
_rng = np.random.default_rng(20261205)
for _ in range(12):   # seeded random shapes (D = 3 takes the element path)
    CASES.append((str(_rng.choice(["bf16", "f32"])), int(_rng.integers(1, 4)), int(_rng.integers(1, 5)),
                  int(_rng.integers(1, 9)), int(_rng.integers(1, 400)), int(_rng.choice([3, 8, 16, 32, 64, 128]))))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-B%d-Hkv%d-rep%d-N%d-D%d" % c)
def test_expand_and_reduce_bitwise(case):
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import gqa
    dtype, B, Hkv, nrep, N, D = case
    H = Hkv * nrep
    say("gqa %s" % (case,))
    k, v, gk, gv = _inputs(torch, B, Hkv, H, N, D, dtype, seed=sum(case[1:]))
    if nrep == 1:
        # the page returns the inputs for equal head counts; the C ABI still copies
        lib = la.load_library()
        ko, vo = torch.empty_like(k), torch.empty_like(v)
        assert lib.la_gqa_expand(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                 ctypes.c_void_p(ko.data_ptr()), ctypes.c_void_p(vo.data_ptr()), B, Hkv,
                                 H, N, D, DT[dtype], None) == 0
        r1, r2 = torch.empty_like(k), torch.empty_like(v)
        assert lib.la_gqa_reduce(ctypes.c_void_p(gk.data_ptr()), ctypes.c_void_p(gv.data_ptr()),
                                 ctypes.c_void_p(r1.data_ptr()), ctypes.c_void_p(r2.data_ptr()), B, Hkv,
                                 H, N, D, DT[dtype], None) == 0
    else:
        ko, vo = gqa.fwd(k, v, Hkv, H)
        r1, r2 = gqa.bwd(gk, gv, Hkv, H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_f64(ko), og.expand(_f64(k), nrep))
    np.testing.assert_array_equal(_f64(vo), og.expand(_f64(v), nrep))
    np.testing.assert_array_equal(_f64(r1), og.round_to(og.reduce(_f64(gk), nrep), dtype))
    np.testing.assert_array_equal(_f64(r2), og.round_to(og.reduce(_f64(gv), nrep), dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_base_and_k_alone(dtype):
    """Bases off 16-byte alignment take the element path; a NULL v pair skips v."""
    torch, la = gpu_or_skip()
    lib = la.load_library()
    B, Hkv, nrep, N, D = 2, 2, 3, 9, 16
    H = Hkv * nrep
    k, _, gk, _ = _inputs(torch, B, Hkv, H, N, D, dtype, seed=4)
    tdt = k.dtype
    buf_in = torch.zeros(k.numel() + 1, dtype=tdt, device="cuda")
    buf_in[1:] = k.reshape(-1)
    kin = buf_in[1:].view(B, Hkv, N, D)                 # one element past a 16-byte boundary
    buf_out = torch.full((B * H * N * D + 1,), 7.0, dtype=tdt, device="cuda")
    kout = buf_out[1:].view(B, H, N, D)
    say("gqa unaligned %s" % dtype)
    assert lib.la_gqa_expand(ctypes.c_void_p(kin.data_ptr()), None, ctypes.c_void_p(kout.data_ptr()), None,
                             B, Hkv, H, N, D, DT[dtype], None) == 0
    gbuf = torch.zeros(gk.numel() + 1, dtype=tdt, device="cuda")
    gbuf[1:] = gk.reshape(-1)
    gin = gbuf[1:].view(B, H, N, D)
    rbuf = torch.full((B * Hkv * N * D + 1,), 7.0, dtype=tdt, device="cuda")
    rout = rbuf[1:].view(B, Hkv, N, D)
    assert lib.la_gqa_reduce(ctypes.c_void_p(gin.data_ptr()), None, ctypes.c_void_p(rout.data_ptr()), None,
                             B, Hkv, H, N, D, DT[dtype], None) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_f64(kout), og.expand(_f64(k), nrep))
    np.testing.assert_array_equal(_f64(rout), og.round_to(og.reduce(_f64(gk), nrep), dtype))
    assert float(buf_out[0]) == 7.0 and float(rbuf[0]) == 7.0   # nothing written before the output


def test_long_gqa_shapes_sampled():
    """B=1, H=32, H_kv=8, N=65536, D=128 bf16 (the benchmark's GQA op shapes),
    in the launch configuration the benchmark times; oracle on sampled rows."""
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import gqa
    c = si.GQA_OPS["gqa_expand_reduce_b1h32kv8n65536d128"]
    B, H, Hkv, N, D = c["B"], c["H"], c["Hkv"], c["N"], c["D"]
    say("gqa long shapes")
    k, v, gk_in, gv_in = _inputs(torch, B, Hkv, H, N, D, c["dtype"], seed=0)
    ko, vo = gqa.fwd(k, v, Hkv, H)
    gk, gv = gqa.bwd(gk_in, gv_in, Hkv, H)
    torch.cuda.synchronize()
    nrep = H // Hkv
    rng = np.random.default_rng(0)
    rows = torch.from_numpy(np.concatenate([rng.integers(0, N, 64), [0, N - 1]])).cuda()
    for h in range(H):
        g = h // nrep
        np.testing.assert_array_equal(_f64(ko[0, h, rows]), _f64(k[0, g, rows]))
        np.testing.assert_array_equal(_f64(vo[0, h, rows]), _f64(v[0, g, rows]))
    for g in range(Hkv):
        sl = slice(g * nrep, (g + 1) * nrep)
        for src, got in ((gk_in, gk), (gv_in, gv)):
            want = og.round_to(og.reduce(_f64(src[0:1, sl][:, :, rows]), nrep), "bf16")[0, 0]
            np.testing.assert_array_equal(_f64(got[0, g, rows]), want)
