"""GPU parity of the low-rank projection (la_lowrank_fwd / la_lowrank_bwd through
linear_attention_transformers_amd.lowrank) against oracle/lowrank.py on the
same seeded inputs.

Tolerance: max |gpu - oracle| / max |oracle| per output <= 2e-2 (bf16
storage; t and g U rounded to bf16 between products, float32 accumulation).
Shapes span ragged edges of every GEMM tile (M, in, rank, out not multiples
of 256; K ranges not multiples of 64), several K splits, leading axes, bias
on and off, plus 16 seeded random shapes; the benchmark's full shapes are
checked on sampled entries;
results are bitwise reproducible."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import lowrank as olr
from parity_util import gpu_or_skip, rel, say

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _t(torch, a):
    return {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16).contiguous() for k, v in a.items()}


def _f64(t):
    return si.exact_f64(t)


CASES = [
    (37, 64, 16, 32, True, None),
    (300, 136, 24, 72, False, None),
    (513, 264, 40, 256, True, None),
    (1, 8, 8, 8, True, None),
    (96, 512, 264, 520, True, None),
    (0, 40, 16, 48, True, (3, 5)),          # leading axes [3, 5]
    (4096, 128, 64, 96, True, None),        # token-axis products in several K splits
]
_rng = np.random.default_rng(20261204)
for _ in range(16):   # seeded random shapes, every dimension ragged against the 256 x 256 x 64 tiles
    CASES.append((int(_rng.integers(1, 5000)), 8 * int(_rng.integers(1, 80)), 8 * int(_rng.integers(1, 48)),
                  8 * int(_rng.integers(1, 80)), bool(_rng.integers(0, 2)), None))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M%d-in%d-r%d-out%d-bias%d-lead%s" % (
    c[0], c[1], c[2], c[3], c[4], "x".join(map(str, c[5])) if c[5] else "no"))
def test_fwd_bwd_against_oracle(case):
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import lowrank
    M, n_in, rank, n_out, with_bias, lead = case
    say("lowrank %s" % (case,))
    a = si.lowrank_draw(M, n_in, rank, n_out, seed=M + n_in, lead=lead)
    t = _t(torch, a)
    bias = t["bias"] if with_bias else None
    y = lowrank.fwd(t["x"], t["U"], t["V"], bias)
    gx, gU, gV, gb = lowrank.bwd(t["x"], t["U"], t["V"], t["grad_out"], bias)
    torch.cuda.synchronize()
    f = {k: _f64(v) for k, v in t.items()}
    yr = olr.fwd(f["x"], f["U"], f["V"], f["bias"] if with_bias else None)
    ref = olr.bwd(f["x"], f["U"], f["V"], f["grad_out"], f["bias"] if with_bias else None)
    assert y.shape == yr.shape
    errs = {"y": rel(_f64(y), yr), "grad_x": rel(_f64(gx), ref[0]), "grad_U": rel(_f64(gU), ref[1]),
            "grad_V": rel(_f64(gV), ref[2])}
    if with_bias:
        errs["grad_bias"] = rel(_f64(gb), ref[3])
    else:
        assert gb is None
    say("  errors %s" % {k: "%.2e" % v for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= TOL, (k, e)


def test_bitwise_reproducible():
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import lowrank
    t = _t(torch, si.lowrank_draw(2048, 256, 64, 128, seed=9))
    outs = []
    for _ in range(2):
        outs.append([lowrank.fwd(t["x"], t["U"], t["V"], t["bias"])] +
                    list(lowrank.bwd(t["x"], t["U"], t["V"], t["grad_out"], t["bias"])))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_autograd_form():
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import lowrank
    t = _t(torch, si.lowrank_draw(64, 32, 16, 24, seed=2))
    leaves = {k: t[k].clone().requires_grad_(True) for k in ("x", "U", "V", "bias")}
    y = lowrank.low_rank_projection(leaves["x"], leaves["U"], leaves["V"], leaves["bias"])
    y.backward(t["grad_out"])
    gx, gU, gV, gb = lowrank.bwd(t["x"], t["U"], t["V"], t["grad_out"], t["bias"])
    for k, ref in (("x", gx), ("U", gU), ("V", gV), ("bias", gb)):
        assert torch.equal(leaves[k].grad, ref)


def test_bench_shapes_sampled():
    """M=32768, in=out=4096, rank=1024 (the benchmark's shapes), in the launch
    configuration it times; the oracle on sampled rows and entries."""
    torch, la = gpu_or_skip()
    from linear_attention_transformers_amd import lowrank
    c = si.LOWRANK_OPS["lowrank_m32768_in4096_r1024_out4096"]
    M, n_in, rank, n_out = c["M"], c["n_in"], c["rank"], c["n_out"]
    say("lowrank bench shapes")
    t = _t(torch, si.lowrank_draw(M, n_in, rank, n_out, seed=0))
    y = lowrank.fwd(t["x"], t["U"], t["V"], t["bias"])
    gx, gU, gV, gb = lowrank.bwd(t["x"], t["U"], t["V"], t["grad_out"], t["bias"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, M, 24), [0, M - 1]])
    x, U, V, b, g = (_f64(t[k]) for k in ("x", "U", "V", "bias", "grad_out"))
    # y and grad_x rows need only their own rows of x and grad_out
    assert rel(_f64(y[rows]), olr.fwd(x[rows], U, V, b)) <= TOL
    gxr = olr.bwd(x[rows], U, V, g[rows], b)[0]
    assert rel(_f64(gx[rows]), gxr) <= TOL
    # grad_U[o, c] = g[:, o] . (x V[c]^T), grad_V[c, i] = (g U[:, c]) . x[:, i], grad_bias: column sums
    cs = rng.integers(0, rank, 4)
    os_ = rng.integers(0, n_out, 6)
    is_ = rng.integers(0, n_in, 6)
    tcol = x @ V[cs].T                     # [M, 4]
    gtcol = g @ U[:, cs]                   # [M, 4]
    refU = g[:, os_].T @ tcol              # [6, 4]
    refV = gtcol.T @ x[:, is_]             # [4, 6]
    assert rel(_f64(gU)[np.ix_(os_, cs)], refU) <= TOL
    assert rel(_f64(gV)[np.ix_(cs, is_)], refV) <= TOL
    assert rel(_f64(gb), g.sum(axis=0)) <= TOL
