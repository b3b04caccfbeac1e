"""The parity gate itself, on the CPU: the per-block normwise gate of
tests/parity_util.py must reject errors that the whole-tensor gate cannot
see at the lengths the kernels run at.

Causal outputs are averages over ever more rows, so their magnitude falls
along the sequence; an error confined to late rows (a segment missing from
later prefixes, a state carry that stops) moves late outputs by many percent
while the whole-tensor ratio, scaled by the first rows, stays under 2e-2.
These cases plant such mistakes in the oracle's own output at the headline
shape (one head, N = 16384, D = 128, elu+1, q, k, v ~ 0.5 N(0,1)) and check
that the whole-tensor gate accepts them and the per-block gate does not.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from parity_util import BLOCK, TOL, block_rel, rel

N, D, SEG = 16384, 128, 512


@pytest.fixture(scope="module")
def headline_unit():
    x = si.draw(1, 1, 1, N, D, 0.5, seed=11, grad=False)
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    out = oracle.fwd(q, k, v, is_causal=True, phi="elu+1", eps=1e-6)
    return q, k, v, out


def dropped_segment(q, k, v, out, s):
    """Outputs with segment s (rows s*SEG .. (s+1)*SEG - 1) missing from the
    prefix of every later row; its own rows and earlier ones unchanged."""
    lo, hi = s * SEG, (s + 1) * SEG
    keep = np.r_[0:lo, hi:N]
    short = oracle.fwd(q[:, :, keep], k[:, :, keep], v[:, :, keep], is_causal=True,
                       phi="elu+1", eps=1e-6)
    mut = out.copy()
    mut[:, :, hi:] = short[:, :, lo:]
    return mut


def test_late_rows_are_small(headline_unit):
    """The premise: the last block's outputs are far smaller than the first's."""
    out = headline_unit[3]
    first = np.max(np.abs(out[..., :BLOCK, :]))
    last = np.max(np.abs(out[..., -BLOCK:, :]))
    assert last < first / 10, (first, last)


@pytest.mark.parametrize("s", [8, 16])
def test_block_gate_catches_dropped_segment(headline_unit, s):
    q, k, v, out = headline_unit
    mut = dropped_segment(q, k, v, out, s)
    whole, blk = rel(mut, out), block_rel(mut, out)
    assert whole <= TOL["bf16"], whole           # the whole-tensor gate is blind to it
    assert blk > 5 * TOL["bf16"], blk            # the per-block gate is not


def test_block_gate_catches_zeroed_late_rows(headline_unit):
    out = headline_unit[3]
    mut = out.copy()
    mut[..., N // 2:, :] = 0.0
    assert rel(mut, out) <= TOL["bf16"]
    assert block_rel(mut, out) >= 0.99


def test_block_gate_accepts_bf16_rounding(headline_unit):
    """Storage rounding of a correct result (2^-9 relative) passes both gates
    with a wide margin."""
    import torch
    out = headline_unit[3]
    r = torch.from_numpy(out).to(torch.bfloat16).double().numpy()
    assert rel(r, out) < 4e-3
    assert block_rel(r, out) < 4e-3


def test_block_gate_zero_blocks():
    """Blocks whose reference is exactly zero (relu rows) are measured against
    the floor, not divided by zero: equal zeros pass, a nonzero fails."""
    ref = np.zeros((1, 1, 2 * BLOCK, 4))
    ref[..., :BLOCK, :] = 1.0
    assert block_rel(ref.copy(), ref) == 0.0
    bad = ref.copy()
    bad[..., BLOCK + 3, 1] = 1e-2
    assert block_rel(bad, ref) > 1.0
