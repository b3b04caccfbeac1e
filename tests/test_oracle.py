"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins.  Sources: SVD_linear_Attention API pages --
'linear_attn' (module docstring: feature maps, chunked causal streaming,
bidirectional reduction, cos/sin modulation; fwd/bwd arguments; bwd is autograd
of fwd) and 'gqa' (bwd: head axis viewed as (H_kv, n_rep), KV gradients summed
over n_rep).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from seeded_inputs import cos_sin, draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
PHIS = ["elu+1", "relu", "identity"]


def rel(a, b):
    """Normwise relative error max|a-b| / max|b|."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def inputs(B, H, Hkv, N, D, seed=0, scale=1.0, positive=False):
    x = draw(B, H, Hkv, N, D, scale, seed)
    if positive:
        x = {n: np.abs(a) for n, a in x.items()}
        x["grad_out"] = draw(B, H, Hkv, N, D, 1.0, seed + 1)["grad_out"]
    return {n: a.astype(np.float64) for n, a in x.items()}


def cs(N):
    c, s = cos_sin(N)
    return c.astype(np.float64), s.astype(np.float64)


# --------------------------------------------------------------------------
# Hand-worked values
# --------------------------------------------------------------------------
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_hand_examples_forward(case):
    q = np.array(case["q"])[None, None]
    k = np.array(case["k"])[None, None]
    v = np.array(case["v"])[None, None]
    cw = np.array(case["cos"]) if "cos" in case else None
    sw = np.array(case["sin"]) if "sin" in case else None
    kw = dict(is_causal=case["causal"], phi=case["phi"], eps=case["eps"],
              cos_weight=cw, sin_weight=sw)
    want = np.array(case["out"])[None, None]
    np.testing.assert_allclose(oracle.fwd(q, k, v, **kw), want, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(oracle.fwd_chunked(q, k, v, 1, **kw), want, rtol=1e-15,
                               atol=1e-15)
    np.testing.assert_allclose(brute.out_np(q, k, v, **kw), want, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("case", _golden()["grad_cases"], ids=lambda c: c["name"])
def test_hand_examples_gradient(case):
    q, k, v, g = (np.array(case[n])[None, None] for n in ("q", "k", "v", "grad_out"))
    kw = dict(is_causal=case["causal"], phi=case["phi"], eps=case["eps"])
    np.testing.assert_allclose(oracle.fwd(q, k, v, **kw), np.array(case["out"])[None, None],
                               rtol=1e-15)
    dq, dk, dv = oracle.bwd(q, k, v, g, **kw)
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        np.testing.assert_allclose(got, np.array(case[name])[None, None], rtol=1e-15,
                                   atol=1e-15)


# --------------------------------------------------------------------------
# P1: recurrent definition == O(N^2) brute force
# --------------------------------------------------------------------------
SHAPES = [(1, 1, 1, 1, 1), (1, 2, 2, 2, 1), (1, 2, 1, 7, 4), (2, 4, 2, 16, 3),
          (1, 3, 3, 33, 8), (1, 8, 2, 20, 4)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("phi", PHIS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_cos", [False, True])
def test_forward_matches_brute_force(shape, phi, causal, use_cos):
    B, H, Hkv, N, D = shape
    x = inputs(B, H, Hkv, N, D, seed=N * 7 + D, positive=(phi == "identity"))
    cw, sw = cs(N) if use_cos else (None, None)
    eps = 1e-6 if phi != "identity" else 0.25
    kw = dict(is_causal=causal, phi=phi, eps=eps, cos_weight=cw, sin_weight=sw)
    got = oracle.fwd(x["q"], x["k"], x["v"], **kw)
    want = brute.out_np(x["q"], x["k"], x["v"], **kw)
    assert rel(got, want) < 1e-12


# --------------------------------------------------------------------------
# P2: chunk algebra == definition, forward and backward, for many chunk sizes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 64, 45, 50])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_cos,phi,hkv", [(False, "elu+1", 2), (True, "relu", 1),
                                              (False, "identity", 2)])
def test_chunked_equals_recurrent(chunk, causal, use_cos, phi, hkv):
    B, H, N, D = 1, 4, 45, 6   # N=45 leaves a ragged last chunk for most sizes
    x = inputs(B, H, hkv, N, D, seed=11, positive=(phi == "identity"))
    cw, sw = cs(N) if use_cos else (None, None)
    kw = dict(is_causal=causal, phi=phi, eps=1e-3, cos_weight=cw, sin_weight=sw)
    o_ref = oracle.fwd(x["q"], x["k"], x["v"], **kw)
    o_ch = oracle.fwd_chunked(x["q"], x["k"], x["v"], chunk, **kw)
    assert rel(o_ch, o_ref) < 1e-12
    g_ref = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], **kw)
    g_ch = oracle.bwd_chunked(x["q"], x["k"], x["v"], x["grad_out"], chunk, **kw)
    for a, b in zip(g_ch, g_ref):
        assert rel(a, b) < 1e-11


# --------------------------------------------------------------------------
# P3: causal row 0 reduces to v_0 (eps = 0) or v_0 s/(s+eps)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("phi", ["elu+1", "relu"])
@pytest.mark.parametrize("use_cos", [False, True])
def test_causal_row0(phi, use_cos):
    B, H, N, D = 2, 4, 9, 5
    x = inputs(B, H, 2, N, D, seed=3)
    cw, sw = cs(N) if use_cos else (None, None)
    out0 = oracle.fwd(x["q"], x["k"], x["v"], True, phi, 0.0, cw, sw)
    kv = np.repeat(np.arange(2), 2)
    v0 = x["v"][:, kv, 0, :]
    qf = brute.phi_np(x["q"][:, :, 0, :], phi)
    kf = brute.phi_np(x["k"][:, kv, 0, :], phi)
    s = np.sum(qf * kf, -1)
    nz = s > 0
    np.testing.assert_allclose(out0[:, :, 0, :][nz], v0[nz], rtol=1e-14, atol=1e-14)
    eps = 0.3
    out_e = oracle.fwd(x["q"], x["k"], x["v"], True, phi, eps, cw, sw)
    np.testing.assert_allclose(out_e[:, :, 0, :], v0 * (s / (s + eps))[..., None],
                               rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P4: outputs lie in the convex hull of the visible v rows (non-negative phi)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("phi", ["elu+1", "relu"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_cos", [False, True])
def test_convex_hull(phi, causal, use_cos):
    B, H, N, D = 1, 2, 40, 3
    x = inputs(B, H, H, N, D, seed=5)
    cw, sw = cs(N) if use_cos else (None, None)
    out = oracle.fwd(x["q"], x["k"], x["v"], causal, phi, 0.0, cw, sw)
    v = x["v"]
    tol = 1e-12
    for i in range(N):
        vis = v[:, :, : i + 1] if causal else v
        lo, hi = vis.min(axis=2), vis.max(axis=2)
        o = out[:, :, i]
        ok = np.isfinite(o)
        assert np.all(o[ok] >= lo[ok] - tol) and np.all(o[ok] <= hi[ok] + tol)
    # with eps > 0 the weights sum to less than one: hull of {0} and the v rows
    out = oracle.fwd(x["q"], x["k"], x["v"], causal, phi, 0.5, cw, sw)
    for i in range(N):
        vis = v[:, :, : i + 1] if causal else v
        lo = np.minimum(vis.min(axis=2), 0.0)
        hi = np.maximum(vis.max(axis=2), 0.0)
        assert np.all(out[:, :, i] >= lo - tol) and np.all(out[:, :, i] <= hi + tol)


# --------------------------------------------------------------------------
# P5: k = 0 with elu+1 gives phi(k) = 1: a running mean (causal) / mean (bidir)
# --------------------------------------------------------------------------
def test_closed_form_running_mean():
    B, H, N, D = 2, 3, 30, 4
    x = inputs(B, H, H, N, D, seed=8)
    k = np.zeros_like(x["k"])
    eps = 1e-2
    s = brute.phi_np(x["q"], "elu+1").sum(-1)                      # [B,H,N]
    cum = np.cumsum(x["v"], axis=2)
    cnt = np.arange(1, N + 1)[None, None, :]
    want = s[..., None] * cum / (cnt * s + eps)[..., None]
    got = oracle.fwd(x["q"], k, x["v"], True, "elu+1", eps)
    assert rel(got, want) < 1e-13
    tot = x["v"].sum(axis=2, keepdims=True)
    want_b = s[..., None] * tot / (N * s + eps)[..., None]
    got_b = oracle.fwd(x["q"], k, x["v"], False, "elu+1", eps)
    assert rel(got_b, want_b) < 1e-13


# --------------------------------------------------------------------------
# P6: identity, eps = 0, bidirectional: (Q (K^T V)) / (Q (K^T 1)) by matmul
# --------------------------------------------------------------------------
def test_identity_bidir_is_two_matmuls():
    B, H, N, D = 2, 2, 50, 7
    x = inputs(B, H, H, N, D, seed=9, positive=True)
    q, k, v = x["q"], x["k"], x["v"]
    num = q @ (np.swapaxes(k, -1, -2) @ v)
    den = q @ k.sum(axis=2)[..., None]
    got = oracle.fwd(q, k, v, False, "identity", 0.0)
    assert rel(got, num / den) < 1e-13


# --------------------------------------------------------------------------
# P7: cos/sin branches == single weighted sum with cos(pi (i-j) / 2N)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("phi", ["elu+1", "relu"])
def test_cosformer_identity(causal, phi):
    B, H, N, D = 1, 2, 24, 5
    x = inputs(B, H, H, N, D, seed=12)
    cw, sw = cs(N)
    got = oracle.fwd(x["q"], x["k"], x["v"], causal, phi, 1e-6, cw, sw)
    i = np.arange(N)
    rho = np.cos(math.pi * (i[:, None] - i[None, :]) / (2.0 * N))
    qf = brute.phi_np(x["q"], phi)
    kf = brute.phi_np(x["k"], phi)
    W = (qf @ np.swapaxes(kf, -1, -2)) * rho
    if causal:
        W = W * np.tril(np.ones((N, N)))
    want = (W @ x["v"]) / (W.sum(-1, keepdims=True) + 1e-6)
    # float32 cos/sin tables vs float64 angles: agreement to float32 rounding
    assert rel(got, want) < 1e-6


# --------------------------------------------------------------------------
# P8: GQA index map h -> h // n_rep (gqa page, bwd: view(B, H_kv, n_rep, N, D))
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_cos", [False, True])
def test_gqa_equals_expanded(causal, use_cos):
    B, H, Hkv, N, D = 2, 6, 2, 13, 4
    nrep = H // Hkv
    x = inputs(B, H, Hkv, N, D, seed=21)
    cw, sw = cs(N) if use_cos else (None, None)
    kw = dict(is_causal=causal, phi="elu+1", eps=1e-6, cos_weight=cw, sin_weight=sw)
    # expansion exactly as the gqa page states it: KV head g feeds query heads
    # g*n_rep .. g*n_rep + n_rep - 1 (repeat-interleave, not tiling)
    ke = np.repeat(x["k"], nrep, axis=1)
    ve = np.repeat(x["v"], nrep, axis=1)
    o_g = oracle.fwd(x["q"], x["k"], x["v"], **kw)
    o_e = oracle.fwd(x["q"], ke, ve, **kw)
    np.testing.assert_array_equal(o_g, o_e)
    dq_g, dk_g, dv_g = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], **kw)
    dq_e, dk_e, dv_e = oracle.bwd(x["q"], ke, ve, x["grad_out"], **kw)
    np.testing.assert_array_equal(dq_g, dq_e)
    # gqa bwd: sum over the n_rep axis of the expanded gradients
    dk_sum = dk_e.reshape(B, Hkv, nrep, N, D).sum(axis=2)
    dv_sum = dv_e.reshape(B, Hkv, nrep, N, D).sum(axis=2)
    assert rel(dk_g, dk_sum) < 1e-13 and rel(dv_g, dv_sum) < 1e-13
    # tiling (h % H_kv) would be a different map: make sure it is not what we do
    kt = np.tile(x["k"], (1, nrep, 1, 1))
    vt = np.tile(x["v"], (1, nrep, 1, 1))
    assert rel(oracle.fwd(x["q"], kt, vt, **kw), o_g) > 1e-3


def test_gqa_locality():
    """Perturbing query head h changes only head h's outputs and KV group h//n_rep."""
    B, H, Hkv, N, D = 1, 4, 2, 10, 3
    x = inputs(B, H, Hkv, N, D, seed=4)
    base = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], True, "elu+1", 1e-6)
    o0 = oracle.fwd(x["q"], x["k"], x["v"], True)
    q2 = x["q"].copy()
    q2[0, 3] += 0.1
    pert = oracle.bwd(q2, x["k"], x["v"], x["grad_out"], True, "elu+1", 1e-6)
    o1 = oracle.fwd(q2, x["k"], x["v"], True)
    for h in range(3):
        np.testing.assert_array_equal(o0[0, h], o1[0, h])
        np.testing.assert_array_equal(base[0][0, h], pert[0][0, h])
    np.testing.assert_array_equal(base[1][0, 0], pert[1][0, 0])
    np.testing.assert_array_equal(base[2][0, 0], pert[2][0, 0])
    assert rel(base[1][0, 1], pert[1][0, 1]) > 0


# --------------------------------------------------------------------------
# P9: gradients -- finite differences and float64 autograd of the brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("phi", PHIS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_cos", [False, True])
def test_gradient_matches_autograd(phi, causal, use_cos):
    B, H, Hkv, N, D = 1, 4, 2, 19, 5
    x = inputs(B, H, Hkv, N, D, seed=31, positive=(phi == "identity"))
    cw, sw = cs(N) if use_cos else (None, None)
    eps = 1e-6 if phi != "identity" else 0.25
    kw = dict(is_causal=causal, phi=phi, eps=eps, cos_weight=cw, sin_weight=sw)
    got = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], **kw)
    want = brute.torch_grads(x["q"], x["k"], x["v"], x["grad_out"], **kw)
    for a, b in zip(got, want):
        assert rel(a, b) < 1e-11


@pytest.mark.parametrize("phi", PHIS)
@pytest.mark.parametrize("causal", [True, False])
def test_gradient_finite_differences(phi, causal):
    B, H, Hkv, N, D = 1, 2, 1, 12, 4
    x = inputs(B, H, Hkv, N, D, seed=41, positive=(phi == "identity"))
    cw, sw = cs(N)
    eps = 1e-3 if phi != "identity" else 0.25
    kw = dict(is_causal=causal, phi=phi, eps=eps, cos_weight=cw, sin_weight=sw)
    g = x["grad_out"]
    grads = oracle.bwd(x["q"], x["k"], x["v"], g, **kw)

    def loss(q, k, v):
        return float(np.sum(oracle.fwd(q, k, v, **kw) * g))

    rng = np.random.default_rng(0)
    names = ("q", "k", "v")
    for t, name in enumerate(names):
        arr = x[name]
        for _ in range(25):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            xv = arr[idx]
            h = 1e-6 * max(1.0, abs(xv))
            if phi == "relu" and name != "v" and abs(xv) < 10 * h:
                continue  # skip the kink of relu
            args = [x[n].copy() for n in names]
            args[t][idx] = xv + h
            up = loss(*args)
            args[t][idx] = xv - h
            dn = loss(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - grads[t][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


# --------------------------------------------------------------------------
# P10: invariants at eps = 0
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_gradient_invariants(causal):
    B, H, Hkv, N, D = 2, 4, 2, 17, 6
    x = inputs(B, H, Hkv, N, D, seed=51)
    g = x["grad_out"]
    nrep = H // Hkv
    for phi in ["relu", "elu+1"]:
        # relu at eps = 0 needs every row to see a positive weight: keep half of
        # each q and k row positive so no denominator is zero
        q, k = x["q"].copy(), x["k"].copy()
        if phi == "relu":
            q[..., : D // 2] = np.abs(q[..., : D // 2])
            k[..., : D // 2] = np.abs(k[..., : D // 2])
        dq, dk, dv = oracle.bwd(q, k, x["v"], g, causal, phi, 0.0)
        # normalised weights sum to one: sum_j dv_j = sum over the group's heads of sum_i g_i
        gsum = g.reshape(B, Hkv, nrep, N, D).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), gsum, rtol=1e-11, atol=1e-11)
        if phi == "relu":
            # scale invariance of each row in q_i and of all k jointly
            np.testing.assert_allclose(np.sum(q * dq, -1), 0.0, atol=1e-11)
            np.testing.assert_allclose(np.sum(k * dk, axis=(2, 3)), 0.0, atol=1e-10)
    # shift invariance: v + u gives out + u
    u = np.linspace(-1, 1, D)
    o1 = oracle.fwd(x["q"], x["k"], x["v"], causal, "elu+1", 0.0)
    o2 = oracle.fwd(x["q"], x["k"], x["v"] + u, causal, "elu+1", 0.0)
    np.testing.assert_allclose(o2 - o1, np.broadcast_to(u, o1.shape), atol=1e-12)


# --------------------------------------------------------------------------
# P11: relu rows with q_i <= 0 give exactly zero output and zero dq
# --------------------------------------------------------------------------
def test_relu_zero_rows():
    B, H, N, D = 1, 2, 16, 4
    x = inputs(B, H, H, N, D, seed=61)
    q = x["q"].copy()
    q[:, :, ::3, :] = -np.abs(q[:, :, ::3, :])
    for causal in (True, False):
        out = oracle.fwd(q, x["k"], x["v"], causal, "relu", 1e-6)
        dq, _, _ = oracle.bwd(q, x["k"], x["v"], x["grad_out"], causal, "relu", 1e-6)
        assert np.all(out[:, :, ::3, :] == 0.0)
        assert np.all(dq[:, :, ::3, :] == 0.0)


# --------------------------------------------------------------------------
# den returned by the forward is Phi(q).z + eps (used by sampled parity checks)
# --------------------------------------------------------------------------
def test_den_output():
    B, H, N, D = 1, 2, 11, 3
    x = inputs(B, H, H, N, D, seed=71)
    _, den = oracle.fwd(x["q"], x["k"], x["v"], True, "elu+1", 0.5, return_den=True)
    W = brute.weights_np(x["q"], x["k"], True, "elu+1")
    np.testing.assert_allclose(den, W.sum(-1) + 0.5, rtol=1e-13)


def test_group_slice_matches_full():
    B, H, Hkv, N, D = 2, 4, 2, 9, 3
    x = inputs(B, H, Hkv, N, D, seed=81)
    full = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], True, "relu", 1e-6)
    q, k, v, g = oracle.group_slice(x["q"], x["k"], x["v"], x["grad_out"], 1, 1)
    part = oracle.bwd(q, k, v, g, True, "relu", 1e-6)
    np.testing.assert_array_equal(part[0][0], full[0][1, 2:4])
    np.testing.assert_array_equal(part[1][0, 0], full[1][1, 1])


def test_rejects_bad_arguments():
    x = inputs(1, 3, 2, 4, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.fwd(x["q"], x["k"], x["v"])  # 3 % 2 != 0
    x = inputs(1, 2, 2, 4, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.fwd(x["q"], x["k"], x["v"], cos_weight=np.ones(4))
