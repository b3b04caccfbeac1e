"""The saved-state backward and the torch.autograd form, through the C ABI.

la_bwd_saved reuses the state records the forward left in the workspace; it
must give exactly la_bwd's gradients on every kernel family.  The autograd
function must return exactly fwd's output and bwd's gradients, which the
parity tests compare with the oracle; one case is compared with the oracle
here as well."""
import pytest

from parity_util import compare, gpu_or_skip, make, oracle_on, say

pytestmark = pytest.mark.gpu

# dtype, D, causal, cos, H, H_kv, N, seg_len: the matrix-core causal,
# bidirectional and cos/sin-GQA paths and the float32 / D = 32 kernels, with
# and without forced segments.  The last case runs its forward on the matrix
# cores and its backward on the float32 kernels (bf16 bidirectional cos/sin),
# whose automatic segmentations differ there (43 and 32 segments).
CASES = [("bf16", 128, True, False, 4, 2, 200, 0), ("bf16", 128, True, False, 4, 2, 200, 64),
         ("bf16", 64, False, False, 4, 4, 150, 64), ("bf16", 128, True, True, 4, 1, 150, 64),
         ("f32", 64, True, False, 2, 1, 130, 64), ("bf16", 32, False, True, 2, 2, 100, 0),
         ("bf16", 64, False, True, 32, 32, 16384, 0),
         # D = 128 with many short segments: the dq kernel walks several
         # segments per workgroup (its multi-segment build)
         ("bf16", 128, True, False, 4, 4, 16300, 64)]


def _id(c):
    return "%s-D%d-%s%s-h%dkv%d-n%d-seg%d" % (c[0], c[1], "causal" if c[2] else "bidir",
                                              "-cos" if c[3] else "", c[4], c[5], c[6], c[7])


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_saved_state_backward_is_bitwise_la_bwd(case):
    torch, la = gpu_or_skip()
    dtype, D, causal, cos, H, Hkv, N, seg_len = case
    say("saved state %s" % _id(case))
    t = make(1, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=7)
    kw = dict(is_causal=causal, phi="elu+1", cos_weight=t["cos_weight"], sin_weight=t["sin_weight"],
              seg_len=seg_len)
    nbytes = la.workspace_bytes("bwd", 1, H, Hkv, N, D, la.LA_BF16 if dtype == "bf16" else la.LA_F32,
                                causal, cos, seg_len)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    la.fwd(t["q"], t["k"], t["v"], workspace=ws, **kw)
    saved = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], workspace=ws, state_from_fwd=True, **kw)
    # twice: the backward leaves the records in place
    again = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], workspace=ws, state_from_fwd=True, **kw)
    ref = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], **kw)
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv"), saved, again, ref):
        assert torch.equal(a, c), name
        assert torch.equal(b, c), name


def test_state_from_fwd_needs_the_workspace():
    torch, la = gpu_or_skip()
    t = make(1, 2, 1, 64, 64, "bf16", seed=1)
    with pytest.raises(ValueError):
        la.bwd(t["q"], t["k"], t["v"], t["grad_out"], is_causal=True, state_from_fwd=True)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        la.bwd(t["q"], t["k"], t["v"], t["grad_out"], is_causal=True, state_from_fwd=True,
               workspace=small)


@pytest.mark.parametrize("case", CASES[:4], ids=[_id(c) for c in CASES[:4]])
def test_autograd_equals_fwd_bwd(case):
    torch, la = gpu_or_skip()
    dtype, D, causal, cos, H, Hkv, N, seg_len = case
    say("autograd %s" % _id(case))
    t = make(1, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=3)
    kw = dict(is_causal=causal, phi="relu", cos_weight=t["cos_weight"], sin_weight=t["sin_weight"],
              seg_len=seg_len)
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = la.linear_attention(q, k, v, **kw)
    out.backward(t["grad_out"])
    ref_out = la.fwd(t["q"], t["k"], t["v"], **kw)
    ref = la.bwd(t["q"], t["k"], t["v"], t["grad_out"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    for name, a, b in zip(("dq", "dk", "dv"), (q.grad, k.grad, v.grad), ref):
        assert torch.equal(a, b), name


def test_autograd_against_the_oracle():
    """GQA, causal, cos/sin weights, bf16: the autograd gradients against the
    fp64 oracle at the bf16 tolerance."""
    torch, la = gpu_or_skip()
    t = make(1, 4, 2, 97, 64, "bf16", scale=0.5, cos=True, seed=11)
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    out = la.linear_attention(q, k, v, is_causal=True, phi="elu+1", cos_weight=t["cos_weight"],
                              sin_weight=t["sin_weight"])
    out.backward(t["grad_out"])
    torch.cuda.synchronize()
    ref = oracle_on(t, True, "elu+1")
    compare(t, out.detach(), (q.grad, k.grad, v.grad), ref[0], ref[1], "bf16", 4, 2,
            label="autograd")
