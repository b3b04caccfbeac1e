"""Pins of the GQA expansion/adjoint oracle (oracle/gqa.py) against what the
gqa page and the mathematics fix, independent of the oracle's own loops:
hand-worked values, NumPy's repeat (a library repeat-interleave), the
adjoint identity <expand(x), y> = <x, reduce(y)>, the linear-attention
oracle's own index mapping, and bf16 rounding ties.  A planted mistake in a
copy of the oracle (tiling map, dropped slot, wrong rounding) fails them."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import gqa as og
from seeded_inputs import draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gqa_examples.json")


def _golden():
    return json.load(open(GOLDEN))


@pytest.mark.parametrize("i", [0, 1])
def test_hand_examples(i):
    c = _golden()["cases"][i]
    np.testing.assert_array_equal(og.expand(np.array(c["k"]), c["n_rep"]), np.array(c["expanded"]))
    np.testing.assert_array_equal(og.reduce(np.array(c["grad"]), c["n_rep"]), np.array(c["reduced"]))


@pytest.mark.parametrize("n_rep", [1, 2, 3, 4, 8])
def test_expand_is_repeat_interleave(n_rep):
    x = draw(2, 3, 3, 5, 4, seed=3)["k"]
    np.testing.assert_array_equal(og.expand(x, n_rep), np.repeat(x.astype(np.float64), n_rep, axis=1))
    # not the tiling map (h % H_kv)
    if n_rep > 1:
        assert not np.array_equal(og.expand(x, n_rep), np.tile(x.astype(np.float64), (1, n_rep, 1, 1)))


@pytest.mark.parametrize("n_rep", [1, 2, 4, 5])
def test_adjoint_identity(n_rep):
    """bwd is the gradient of fwd: <expand(x), y> = <x, reduce(y)> for all x, y."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 6, 4))
    y = rng.standard_normal((2, 3 * n_rep, 6, 4))
    lhs = np.sum(og.expand(x, n_rep) * y)
    rhs = np.sum(x * og.reduce(y, n_rep))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # and per element: d<expand(x), y>/dx[b, g] = sum over the group's slots
    for g in range(3):
        np.testing.assert_allclose(og.reduce(y, n_rep)[:, g], y[:, g * n_rep:(g + 1) * n_rep].sum(axis=1),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_rep", [2, 4, 8])
def test_reduce_of_expand(n_rep):
    x = draw(1, 2, 2, 7, 8, seed=5)["v"].astype(np.float64)
    np.testing.assert_array_equal(og.reduce(og.expand(x, n_rep), n_rep), n_rep * x)


def test_matches_linear_attention_index_map():
    """The attention oracle with H_kv < H equals it on expanded k, v; its dk, dv
    equal reduce() of the expanded run's (the gqa page read by both modules)."""
    B, H, Hkv, N, D = 1, 4, 2, 9, 4
    n_rep = H // Hkv
    x = draw(B, H, Hkv, N, D, seed=11)
    kw = dict(is_causal=True, phi="relu", eps=1e-6)
    ke, ve = og.expand(x["k"], n_rep), og.expand(x["v"], n_rep)
    np.testing.assert_array_equal(oracle.fwd(x["q"], x["k"], x["v"], **kw), oracle.fwd(x["q"], ke, ve, **kw))
    _, dk, dv = oracle.bwd(x["q"], x["k"], x["v"], x["grad_out"], **kw)
    _, dke, dve = oracle.bwd(x["q"], ke, ve, x["grad_out"], **kw)
    np.testing.assert_allclose(og.reduce(dke, n_rep), dk, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(og.reduce(dve, n_rep), dv, rtol=1e-12, atol=1e-14)


def test_bf16_rounding_ties():
    pairs = _golden()["bf16_rounding"]["pairs"]
    a = np.array([p[0] for p in pairs])
    np.testing.assert_array_equal(og.round_to(a, "bf16"), np.array([p[1] for p in pairs]))


def test_bf16_rounding_matches_library_on_float32_values():
    """On values that are exactly float32, one rounding float64 -> bf16 is the
    library's float32 -> bf16 conversion (nearest even)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
                        np.float32([0.0, -0.0, 1e-45, 3.0e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(og.round_to(x.astype(np.float64), "bf16"), ref)


def test_f32_rounding_is_one_rounding():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, -(1.0 + 2.0 ** -23 + 2.0 ** -30)])
    np.testing.assert_array_equal(og.round_to(x, "f32"), [1.0, 1.0 + 2.0 ** -22, -(1.0 + 2.0 ** -23)])


MUTANTS = {
    "tiling": lambda x, n: np.tile(np.asarray(x, np.float64), (1, n, 1, 1)),
    "dropped_slot": lambda x, n: np.concatenate([og.expand(x, n)[:, :-1], np.zeros_like(og.expand(x, n)[:, :1])], axis=1),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutated_expand(name):
    bad = MUTANTS[name]
    c = _golden()["cases"][0]
    caught = not np.array_equal(bad(np.array(c["k"]), c["n_rep"]), np.array(c["expanded"]))
    x = draw(1, 2, 2, 3, 4, seed=1)["k"]
    caught_lib = not np.array_equal(bad(x, 2), np.repeat(x.astype(np.float64), 2, axis=1))
    assert caught and caught_lib


def test_pins_reject_mutated_rounding():
    truncate = lambda x: np.ldexp(np.trunc(np.ldexp(np.frexp(x)[0], 8)), np.frexp(x)[1] - 8)
    half_up = lambda x: np.ldexp(np.floor(np.ldexp(np.frexp(x)[0], 8) + 0.5), np.frexp(x)[1] - 8)
    pairs = _golden()["bf16_rounding"]["pairs"]
    a, want = np.array([p[0] for p in pairs]), np.array([p[1] for p in pairs])
    assert not np.array_equal(truncate(a), want)
    assert not np.array_equal(half_up(a), want)
