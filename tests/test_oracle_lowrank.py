"""Pins of the low-rank projection oracle (oracle/lowrank.py) against what the
low_rank page and the mathematics fix: hand-worked values, central finite
differences of fwd for every gradient, the identity projection, the other
association order x (U V)^T, and planted mistakes that those pins reject."""
import json
import os

import numpy as np
import pytest

from oracle import lowrank as olr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lowrank_examples.json")


def _g():
    return json.load(open(GOLDEN))


@pytest.mark.parametrize("which", ["first", "second"])
def test_hand_examples(which):
    c = _g() if which == "first" else _g()["second"]
    a = {k: np.array(v) for k, v in c.items() if k not in ("note", "citation", "second")}
    np.testing.assert_array_equal(olr.fwd(a["x"], a["U"], a["V"], a["bias"]), a["y"])
    gx, gU, gV, gb = olr.bwd(a["x"], a["U"], a["V"], a["grad_out"], a["bias"])
    np.testing.assert_array_equal(gx, a["grad_x"])
    np.testing.assert_array_equal(gU, a["grad_U"])
    np.testing.assert_array_equal(gV, a["grad_V"])
    np.testing.assert_array_equal(gb, a["grad_bias"])


def _rand(seed, M=5, n_in=6, r=3, n_out=4, lead=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((*(lead or (M,)), n_in))
    return (x, rng.standard_normal((n_out, r)), rng.standard_normal((r, n_in)),
            rng.standard_normal(n_out), rng.standard_normal((*(lead or (M,)), n_out)))


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("lead", [None, (2, 3)])
def test_gradients_match_finite_differences(with_bias, lead):
    x, U, V, b, g = _rand(3, lead=lead)
    b = b if with_bias else None
    L = lambda x_, U_, V_, b_: float(np.sum(olr.fwd(x_, U_, V_, b_) * g))
    grads = olr.bwd(x, U, V, g, b)
    h = 1e-6
    for idx, arr in enumerate([x, U, V] + ([b] if with_bias else [])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = [x.copy(), U.copy(), V.copy(), None if b is None else b.copy()]
            args[idx][i] += h
            up = L(*args)
            args[idx][i] -= 2 * h
            dn = L(*args)
            num[i] = (up - dn) / (2 * h)
        np.testing.assert_allclose(grads[idx], num, rtol=1e-7, atol=1e-7)
    if not with_bias:
        assert grads[3] is None


def test_identity_projection():
    rng = np.random.default_rng(4)
    x, b = rng.standard_normal((7, 5)), rng.standard_normal(5)
    I = np.eye(5)
    np.testing.assert_array_equal(olr.fwd(x, I, I, b), x + b)
    g = rng.standard_normal((7, 5))
    gx, gU, gV, gb = olr.bwd(x, I, I, g, b)
    np.testing.assert_array_equal(gx, g)
    np.testing.assert_allclose(gU, g.T @ x, rtol=1e-14)
    np.testing.assert_allclose(gb, g.sum(axis=0), rtol=1e-14)


def test_other_association_order():
    """(x V^T) U^T = x (U V)^T: the product of the two factors applied at once."""
    x, U, V, b, _ = _rand(5, M=9, n_in=8, r=2, n_out=6)
    np.testing.assert_allclose(olr.fwd(x, U, V, b), x @ (U @ V).T + b, rtol=1e-12, atol=1e-12)


def _fd_grads(x, U, V, b, g, h=1e-6):
    """Central finite differences of sum(fwd * g) for x, U, V, b."""
    L = lambda *a: float(np.sum(olr.fwd(*a) * g))
    out = []
    for idx, arr in enumerate([x, U, V, b]):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            args = [x.copy(), U.copy(), V.copy(), b.copy()]
            args[idx][it.multi_index] += h
            up = L(*args)
            args[idx][it.multi_index] -= 2 * h
            num[it.multi_index] = (up - L(*args)) / (2 * h)
        out.append(num)
    return out


def test_pins_reject_planted_mistakes():
    """Plausible mistakes in a copy of the oracle fail the pins above."""
    c = _g()
    a = {k: np.array(v) for k, v in c.items() if k not in ("note", "citation", "second")}
    # forward: bias dropped (hand example), U untransposed or factors swapped
    # (square factors keep both well-formed; the other-order identity catches them)
    assert not np.array_equal((a["x"] @ a["V"].T) @ a["U"].T, a["y"])
    rng = np.random.default_rng(8)
    x, U, V, b = (rng.standard_normal((4, 3)), rng.standard_normal((3, 3)),
                  rng.standard_normal((3, 3)), rng.standard_normal(3))
    good = x @ (U @ V).T + b
    assert not np.allclose((x @ V.T) @ U + b, good)
    assert not np.allclose((x @ U.T) @ V.T + b, good)
    # backward: transposed grad_U, grad_t from U^T, grad_V from t: finite differences reject each
    g = rng.standard_normal((4, 3))
    fd = _fd_grads(x, U, V, b, g)
    t = x @ V.T
    assert not np.allclose(t.T @ g, fd[1], atol=1e-6)                 # grad_U transposed
    assert not np.allclose((g @ U.T) @ V, fd[0], atol=1e-6)           # grad_t = g U^T
    assert not np.allclose((g @ U).T @ t, fd[2], atol=1e-6)           # grad_V from t, not x
    np.testing.assert_allclose(olr.bwd(x, U, V, g, b)[1], fd[1], atol=1e-7)   # the oracle passes
