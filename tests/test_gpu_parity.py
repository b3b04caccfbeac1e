"""GPU parity: the HIP path (through the C ABI and its binding) against the
CPU oracle on the same seeded inputs.

* small shapes that span several chunks, several segments and a ragged tail,
  for every storage type, head size, feature map, mode, cos/sin and GQA;
* edge cases (N = 1, N shorter than a chunk, one row past a chunk boundary);
* 64 seeded random configurations, every argument drawn at once (storage
  type, D, feature map, mode, cos/sin, B, H, H_kv, ragged N, segment length,
  saved or recomputed state);
* the five specified workloads at full size in the launch configuration the
  benchmark times, compared on sampled (batch, KV head) groups, which the
  oracle computes exactly because groups never interact;
* GQA index mapping: bitwise equal to a pre-expanded run (out, dq), and local
  (perturbing one query head changes nothing else) -- gqa page, bwd;
* run-to-run bitwise determinism.
"""
import numpy as np
import pytest

import seeded_inputs as si
from parity_util import compare, gpu_or_skip, make, np64, oracle_on, run_gpu, say

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# small shapes, full oracle
# --------------------------------------------------------------------------
SMALL = []
for dtype in ("f32", "bf16"):
    for D in (32, 64, 128):
        for phi in ("elu+1", "relu"):
            for causal in (True, False):
                SMALL.append((dtype, D, phi, causal, False, 4, 2))
    for D in (32, 64, 128):
        SMALL.append((dtype, D, "elu+1", True, True, 4, 1))
        SMALL.append((dtype, D, "relu", False, True, 2, 2))
    SMALL.append((dtype, 64, "identity", True, False, 2, 2))
    SMALL.append((dtype, 64, "identity", False, True, 4, 4))


def _id(c):
    dtype, D, phi, causal, cos, H, Hkv = c
    return "%s-D%d-%s-%s%s-h%dkv%d" % (dtype, D, phi, "causal" if causal else "bidir",
                                       "-cos" if cos else "", H, Hkv)


@pytest.mark.parametrize("case", SMALL, ids=[_id(c) for c in SMALL])
def test_small_shapes(case):
    torch, la = gpu_or_skip()
    dtype, D, phi, causal, cos, H, Hkv = case
    B, N = 2, 300                     # 300 rows: several chunks, ragged tail
    positive = phi == "identity"
    t = make(B, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=D + H)
    if positive:   # identity is not non-negative: keep the denominators away from 0
        for n in ("q", "k"):
            t[n] = t[n].abs()
    eps = 1e-6 if not positive else 1.0
    say("case %s" % _id(case))
    ref = oracle_on(t, causal, phi, eps)
    for seg_len in (0, 64):           # automatic split, then many short segments
        out, grads = run_gpu(la, t, causal, phi, eps, seg_len=seg_len)
        compare(t, out, grads, ref[0], ref[1], dtype, H, Hkv, label="%s-seg%d" % (_id(case), seg_len))


# --------------------------------------------------------------------------
# seeded random configurations: every argument drawn at once, so that
# combinations the grids above do not list (GQA with cos/sin in float32 at
# D = 32, identity with a forced segment length, the saved-state backward on
# ragged N, ...) are also run against the oracle
# --------------------------------------------------------------------------
def _random_cases(count=64, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        Hkv = int(rng.integers(1, 3))
        cases.append(dict(
            dtype=str(rng.choice(["bf16", "f32"])), D=int(rng.choice([32, 64, 128])),
            phi=str(rng.choice(["elu+1", "relu", "identity"])), causal=bool(rng.integers(0, 2)),
            cos=bool(rng.integers(0, 2)), B=int(rng.integers(1, 3)), Hkv=Hkv,
            H=Hkv * int(rng.integers(1, 4)), N=int(rng.integers(1, 701)),
            seg_len=int(rng.choice([0, 64, 128, 192])), saved=bool(rng.integers(0, 2)), seed=1000 + i))
    return cases


RANDOM = _random_cases()


def _rid(c):
    return "%s-D%d-%s-%s%s-b%dh%dkv%d-n%d-seg%d%s" % (
        c["dtype"], c["D"], c["phi"], "causal" if c["causal"] else "bidir", "-cos" if c["cos"] else "",
        c["B"], c["H"], c["Hkv"], c["N"], c["seg_len"], "-saved" if c["saved"] else "")


@pytest.mark.parametrize("c", RANDOM, ids=[_rid(c) for c in RANDOM])
def test_random_configurations(c):
    torch, la = gpu_or_skip()
    t = make(c["B"], c["H"], c["Hkv"], c["N"], c["D"], c["dtype"], scale=0.5, cos=c["cos"], seed=c["seed"])
    positive = c["phi"] == "identity"
    if positive:   # identity is not non-negative: keep the denominators away from 0
        for n in ("q", "k"):
            t[n] = t[n].abs()
    eps = 1.0 if positive else 1e-6
    say("case %s" % _rid(c))
    ref = oracle_on(t, c["causal"], c["phi"], eps)
    out, grads = run_gpu(la, t, c["causal"], c["phi"], eps, seg_len=c["seg_len"], saved=c["saved"])
    compare(t, out, grads, ref[0], ref[1], c["dtype"], c["H"], c["Hkv"], label=_rid(c))


@pytest.mark.parametrize("N", [1, 5, 31, 33, 64, 65, 129])
@pytest.mark.parametrize("causal", [True, False])
def test_edge_lengths(N, causal):
    torch, la = gpu_or_skip()
    for dtype, D, cos in (("f32", 64, False), ("bf16", 128, False), ("bf16", 128, True)):
        t = make(1, 2, 1, N, D, dtype, scale=0.5, cos=cos, seed=N)
        # with one row and a tiny eps, out = v exactly up to eps and dq, dk are
        # O(eps): a normwise comparison would measure rounding noise only
        eps = 0.5 if N == 1 else 1e-6
        say("edge N=%d %s D=%d cos=%s causal=%s eps=%g" % (N, dtype, D, cos, causal, eps))
        ref = oracle_on(t, causal, "elu+1", eps)
        out, grads = run_gpu(la, t, causal, "elu+1", eps)
        compare(t, out, grads, ref[0], ref[1], dtype, 2, 1, label="edge-N%d-%s-D%d%s-%s" % (
            N, dtype, D, "-cos" if cos else "", "causal" if causal else "bidir"),
            grad_blocks=N > 1)


@pytest.mark.parametrize("D", [64, 128])
def test_bidir_cos_gqa_many_segments(D):
    """The bidirectional cos/sin backward on the matrix cores: GQA (n_rep = 4),
    elu+1, 1100 rows (a ragged tail), at the automatic split and with a
    segment boundary every 64 rows (17 per-segment records in each scan)."""
    torch, la = gpu_or_skip()
    B, H, Hkv, N = 1, 8, 2, 1100
    t = make(B, H, Hkv, N, D, "bf16", scale=0.5, cos=True, seed=40 + D)
    say("bidir cos gqa D=%d" % D)
    ref = oracle_on(t, False, "elu+1")
    for seg_len in (0, 64):
        out, grads = run_gpu(la, t, False, "elu+1", seg_len=seg_len)
        compare(t, out, grads, ref[0], ref[1], "bf16", H, Hkv,
                label="bidir-cos-gqa-D%d-seg%d" % (D, seg_len))


MANYSEG = [("f32", 32, True, False), ("f32", 32, False, False), ("f32", 64, False, False),
           ("f32", 128, False, False), ("bf16", 64, False, False), ("bf16", 64, True, False),
           ("bf16", 64, True, True), ("bf16", 128, True, True)]


@pytest.mark.parametrize("dtype,D,causal,cos", MANYSEG,
                         ids=["%s-D%d-%s%s" % (d, D, "causal" if c else "bidir", "-cos" if w else "")
                              for d, D, c, w in MANYSEG])
def test_many_segments_every_family(dtype, D, causal, cos):
    """18 segments of 64 rows (N = 1100): the segment scans then load their
    records in more than one batch, in both modes and on every kernel family
    (float32 vector-ALU at D = 32, float32 matrix cores, bf16 matrix cores,
    and the causal cos/sin kernels with their R-record pass); GQA with
    n_rep = 2."""
    torch, la = gpu_or_skip()
    B, H, Hkv, N = 1, 4, 2, 1100
    t = make(B, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=D + N + cos)
    say("many segments %s D=%d causal=%s cos=%s" % (dtype, D, causal, cos))
    ref = oracle_on(t, causal, "relu", 1e-6)
    out, grads = run_gpu(la, t, causal, "relu", 1e-6, seg_len=64)
    compare(t, out, grads, ref[0], ref[1], dtype, H, Hkv, label="manyseg-%s-D%d-%s%s" % (
        dtype, D, "causal" if causal else "bidir", "-cos" if cos else ""))


COS_HEADS = [(3, 1, 0), (3, 1, 64), (2, 2, 64), (5, 1, 0)]


@pytest.mark.parametrize("H,Hkv,seg_len", COS_HEADS,
                         ids=["h%dkv%d-seg%d" % c for c in COS_HEADS])
def test_causal_cos_head_counts(H, Hkv, seg_len):
    """The causal cos/sin kernels (D = 128, F = 256) at odd and single head
    counts per KV head: n_rep = 3 and 5 (the forward's per-head buffers then
    end a chunk on the buffer the next chunk's first head takes) and
    n_rep = 1; a ragged N = 700 over several 32-row chunks per segment, at
    the automatic split and at 64-row segments."""
    torch, la = gpu_or_skip()
    B, N, D = 1, 700, 128
    t = make(B, H, Hkv, N, D, "bf16", scale=0.5, cos=True, seed=H + 10 * Hkv + seg_len)
    say("causal cos heads H=%d Hkv=%d seg_len=%d" % (H, Hkv, seg_len))
    ref = oracle_on(t, True, "elu+1", 1e-6)
    out, grads = run_gpu(la, t, True, "elu+1", 1e-6, seg_len=seg_len)
    compare(t, out, grads, ref[0], ref[1], "bf16", H, Hkv, label="cos-heads-h%dkv%d-seg%d" % (H, Hkv, seg_len))


GROUPED = [("bf16", 64, False), ("bf16", 128, False), ("bf16", 64, True), ("f32", 64, False)]


@pytest.mark.parametrize("dtype,D,cos", GROUPED,
                         ids=["%s-D%d%s" % (d, D, "-cos" if c else "") for d, D, c in GROUPED])
def test_bidir_dkdv_grouped_segments(dtype, D, cos):
    """Bidirectional dk/dv workgroups that walk several segments: 16 (batch,
    KV head) units of 17 segments of 64 rows (N = 1070, ragged) give the bf16
    F = D kernel 16 workgroups per unit, two segments each and the last one a
    single segment; GQA n_rep = 2.  The cos/sin and float32 dk/dv kernels run
    one segment per workgroup on the same shape."""
    torch, la = gpu_or_skip()
    B, H, Hkv, N = 2, 16, 8, 1070
    t = make(B, H, Hkv, N, D, dtype, scale=0.5, cos=cos, seed=D + N + cos)
    say("grouped dk/dv %s D=%d cos=%s" % (dtype, D, cos))
    ref = oracle_on(t, False, "elu+1", 1e-6)
    out, grads = run_gpu(la, t, False, "elu+1", 1e-6, seg_len=64)
    compare(t, out, grads, ref[0], ref[1], dtype, H, Hkv, label="grouped-%s-D%d%s" % (
        dtype, D, "-cos" if cos else ""))


SPAN = [(128, True, 4, 4, 16300), (128, False, 8, 4, 16300), (128, True, 8, 2, 16300),
        (64, False, 8, 8, 32000)]


@pytest.mark.parametrize("D,causal,H,Hkv,N", SPAN,
                         ids=["D%d-%s-h%dkv%d-n%d" % (D, "causal" if c else "bidir", H, Hkv, N)
                              for D, c, H, Hkv, N in SPAN])
def test_dq_workgroup_spans_segments(D, causal, H, Hkv, N):
    """Many short segments (seg_len 64) over a long ragged sequence, where the
    dq kernel runs one workgroup per compute unit at D = 128: it then walks
    several consecutive segments per workgroup (its state carry crosses their
    boundaries) and writes one (R, r) record per segment.  The D = 64
    bidirectional case (8 units x 500 segments) also has each dk/dv
    workgroup walk 16 segments."""
    torch, la = gpu_or_skip()
    B = 1
    t = make(B, H, Hkv, N, D, "bf16", scale=0.5, cos=False, seed=D + H + N)
    say("span D=%d causal=%s H=%d Hkv=%d N=%d seg_len=64" % (D, causal, H, Hkv, N))
    ref = oracle_on(t, causal, "elu+1", 1e-6)
    out, grads = run_gpu(la, t, causal, "elu+1", 1e-6, seg_len=64, saved=True)
    compare(t, out, grads, ref[0], ref[1], "bf16", H, Hkv, label="span-D%d-%s-h%dkv%d" % (
        D, "causal" if causal else "bidir", H, Hkv))


def test_tiny_fp32_workload():
    """B=1, H=2, N=256, D=32, float32, elu+1, eps=1e-6, both modes, fwd+bwd."""
    torch, la = gpu_or_skip()
    w = si.WORKLOADS["tiny_fp32"]
    t = si.workload_inputs(w, "f32", "cuda")
    for mode in w.modes:
        causal = mode == "causal"
        ref = oracle_on(t, causal, w.phi, w.eps)
        for seg_len in (0, 64):
            say("tiny_fp32 %s seg_len=%d" % (mode, seg_len))
            out, grads = run_gpu(la, t, causal, w.phi, w.eps, seg_len=seg_len)
            compare(t, out, grads, ref[0], ref[1], "f32", w.H, w.Hkv,
                    label="tiny_fp32-%s-seg%d" % (mode, seg_len))


# --------------------------------------------------------------------------
# full-size workloads, sampled groups
# --------------------------------------------------------------------------
def _sample_groups(w, count):
    rng = np.random.default_rng(123)
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    idx = sorted(rng.choice(len(units), size=min(count, len(units)), replace=False))
    # always include the first and the last group
    pick = {units[0], units[-1]} | {units[i] for i in idx}
    return sorted(pick)[:max(count, 2)]


FULL = [("causal_fwd_b4h16n4096d64", "bf16", 6), ("bidir_enc_b16h12n2048d64", "bf16", 6),
        ("bidir_enc_b16h12n2048d64", "f32", 6), ("causal_train_b2h32n16384d128", "bf16", 4),
        ("causal_gqa_cos_b1h32kv8n65536d128", "bf16", 1)]


@pytest.mark.parametrize("name,dtype,count", FULL, ids=["%s-%s" % (n, d) for n, d, _ in FULL])
def test_full_size_workloads(name, dtype, count):
    """The benchmark's launch configuration: one workspace for la_fwd and the
    backward on its state records (la_bwd_saved), gated whole and per block of
    rows on sampled groups; then la_bwd (state computed again) must give the
    same gradients bit for bit."""
    torch, la = gpu_or_skip()
    w = si.WORKLOADS[name]
    say("workload %s %s: drawing inputs" % (name, dtype))
    t = si.workload_inputs(w, dtype, "cuda")
    causal = w.modes == ("causal",)
    say("workload %s %s: GPU run (saved-state backward)" % (name, dtype))
    out, grads = run_gpu(la, t, causal, w.phi, w.eps, backward=w.backward, saved=w.backward)
    groups = _sample_groups(w, count)
    say("workload %s: oracle on groups %s" % (name, groups))
    ref = oracle_on(t, causal, w.phi, w.eps, backward=w.backward, groups=groups)
    compare(t, out, grads, ref[0], ref[1], dtype, w.H, w.Hkv, groups=groups,
            label="%s-%s" % (name, dtype))
    # every output is finite everywhere, not only on the sampled groups
    assert torch.isfinite(out).all()
    if grads is not None:
        assert all(torch.isfinite(x).all() for x in grads)
        say("workload %s: la_bwd (state computed again) against the saved-state run" % name)
        _, again = run_gpu(la, t, causal, w.phi, w.eps, backward=True, saved=False)
        for n, a, b in zip(("dq", "dk", "dv"), grads, again):
            assert torch.equal(a, b), n


# --------------------------------------------------------------------------
# GQA head-index mapping (gqa page, bwd: head axis viewed as (H_kv, n_rep))
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_bitwise_equals_expanded(dtype, causal):
    torch, la = gpu_or_skip()
    B, H, Hkv, N, D = 2, 8, 2, 200, 64
    nrep = H // Hkv
    t = make(B, H, Hkv, N, D, dtype, scale=0.5, cos=True, seed=7)
    e = dict(t)
    e["k"] = t["k"].repeat_interleave(nrep, dim=1).contiguous()
    e["v"] = t["v"].repeat_interleave(nrep, dim=1).contiguous()
    out_g, (dq_g, dk_g, dv_g) = run_gpu(la, t, causal, "relu")
    out_e, (dq_e, dk_e, dv_e) = run_gpu(la, e, causal, "relu")
    assert torch.equal(out_g, out_e)
    assert torch.equal(dq_g, dq_e)
    # KV gradients: sum over the n_rep axis of the expanded gradients
    dk_sum = dk_e.float().view(B, Hkv, nrep, N, D).sum(2)
    dv_sum = dv_e.float().view(B, Hkv, nrep, N, D).sum(2)
    tol = 1e-4 if dtype == "f32" else 2e-2
    for a, b in ((dk_g, dk_sum), (dv_g, dv_sum)):
        err = (a.float() - b).abs().max() / b.abs().max()
        assert err <= tol, float(err)


def test_gqa_locality():
    torch, la = gpu_or_skip()
    B, H, Hkv, N, D = 1, 8, 2, 150, 32
    t = make(B, H, Hkv, N, D, "f32", seed=9)
    base_out, base_g = run_gpu(la, t, True, "elu+1")
    p = dict(t)
    p["q"] = t["q"].clone()
    p["q"][0, 5] += 0.25                      # query head 5 -> KV head 5 // 4 = 1
    out, grads = run_gpu(la, p, True, "elu+1")
    for h in range(H):
        if h != 5:
            assert torch.equal(out[0, h], base_out[0, h])
            assert torch.equal(grads[0][0, h], base_g[0][0, h])
    assert torch.equal(grads[1][0, 0], base_g[1][0, 0])   # other KV head untouched
    assert torch.equal(grads[2][0, 0], base_g[2][0, 0])
    assert not torch.equal(grads[1][0, 1], base_g[1][0, 1])


def test_deterministic():
    torch, la = gpu_or_skip()
    t = make(2, 4, 2, 1000, 128, "bf16", scale=0.5, cos=True, seed=3)
    a_out, a_g = run_gpu(la, t, True, "relu")
    b_out, b_g = run_gpu(la, t, True, "relu")
    assert torch.equal(a_out, b_out)
    for x, y in zip(a_g, b_g):
        assert torch.equal(x, y)


def test_zero_rows_relu_exact():
    """relu rows whose q is all <= 0 give exactly zero output and dq."""
    torch, la = gpu_or_skip()
    t = make(1, 2, 2, 100, 64, "f32", seed=5)
    t["q"][:, :, ::7] = -t["q"][:, :, ::7].abs()
    out, (dq, _, _) = run_gpu(la, t, True, "relu")
    assert torch.count_nonzero(out[:, :, ::7]) == 0
    assert torch.count_nonzero(dq[:, :, ::7]) == 0


def test_binding_errors_on_gpu():
    torch, la = gpu_or_skip()
    q = torch.zeros(1, 3, 16, 32, device="cuda")
    k = torch.zeros(1, 2, 16, 32, device="cuda")
    with pytest.raises(ValueError):
        la.fwd(q, k, k)                                   # 3 % 2 != 0
    q = torch.zeros(1, 2, 16, 48, device="cuda")
    with pytest.raises(ValueError):
        la.fwd(q, q, q)                                   # D = 48 unsupported
    q = torch.zeros(1, 2, 16, 32, device="cuda", dtype=torch.float16)
    with pytest.raises(ValueError):
        la.fwd(q, q, q)                                   # fp16 storage not served
    q = torch.zeros(1, 2, 16, 32, device="cuda")
    with pytest.raises(ValueError):
        la.fwd(q, q, q, cos_weight=torch.ones(16, device="cuda"))


def test_kernel_family_per_case():
    """bf16 runs on the matrix-core kernels (causal and bidirectional, forward
    and backward, with and without cos/sin); float32 bidirectional
    without cos/sin at D = 64 and 128 on the float32 matrix-core kernels, other
    float32 cases on
    the vector-ALU kernels (checked through the library's launch timing)."""
    torch, la = gpu_or_skip()
    t = make(1, 4, 2, 600, 128, "bf16", scale=0.5, seed=1)   # three 256-row segments
    la.timing_enable(True)
    try:
        run_gpu(la, t, True, "elu+1", backward=False)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert "k_fwd_mfma" in names and "k_state_mfma" in names, names
    # one segment: a causal pass needs no segment sums (its prefix is zero)
    t = make(1, 4, 2, 256, 128, "bf16", scale=0.5, seed=1)
    la.timing_enable(True)
    try:
        run_gpu(la, t, True, "elu+1", backward=False)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert "k_fwd_mfma" in names and "k_state_mfma" not in names, names
    t = make(1, 4, 2, 256, 128, "f32", seed=1)
    la.timing_enable(True)
    try:
        run_gpu(la, t, True, "elu+1", backward=False)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert "k_fwd_causal" in names, names
    t = make(1, 4, 2, 256, 64, "bf16", seed=1)
    la.timing_enable(True)
    try:
        run_gpu(la, t, False, "relu", backward=True)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert {"k_state_mfma", "k_fwd_bidir_mfma", "k_bwd_q_bidir_mfma", "k_bwd_kv_bidir_mfma"} <= names, names
    t = make(1, 4, 2, 256, 64, "bf16", cos=True, scale=0.5, seed=1)
    la.timing_enable(True)
    try:
        run_gpu(la, t, True, "relu", backward=True)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert {"k_bwd_q_cos_mfma", "k_bwd_r_cos_mfma", "k_bwd_kv_cos_mfma"} <= names, names
    t = make(1, 4, 2, 300, 128, "bf16", cos=True, seed=3)
    la.timing_enable(True)
    try:
        run_gpu(la, t, False, "relu", backward=True)
        names = set(la.timing_collect())
    finally:
        la.timing_enable(False)
    assert {"k_bwd_q_cos_bidir_mfma", "k_bwd_r_cos_bidir_mfma", "k_bwd_kv_cos_bidir_mfma"} <= names, names
    for D in (64, 128):
        t = make(1, 4, 2, 300, D, "f32", seed=2)
        la.timing_enable(True)
        try:
            run_gpu(la, t, False, "elu+1", backward=True)
            names = set(la.timing_collect())
        finally:
            la.timing_enable(False)
        assert {"k_state_f32", "k_fwd_bidir_f32", "k_bwd_q_bidir_f32",
                "k_bwd_kv_bidir_f32"} <= names, (D, names)
