"""The oracle's pins have teeth: plant a plausible mistake in a copy of the C
oracle (on the CPU), rebuild it, and check that the pins reject the copy.

Each mutation is a textual edit of ``oracle/linattn_oracle.c``; the pins used
are the independent ones of ``test_oracle.py`` (hand-worked values, the O(N^2)
brute force, float64 autograd, the gqa page's expand/sum semantics).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from seeded_inputs import cos_sin, draw

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "linattn_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")

MUTATIONS = {
    "eps_dropped": ("        double den = eps;\n                for (int f = 0; f < F; ++f) "
                    "den += qf[f] * z[f];",
                    "        double den = 0.0;\n                for (int f = 0; f < F; ++f) "
                    "den += qf[f] * z[f];"),
    "elu_without_plus_one": ("return x > 0.0 ? x + 1.0 : exp(x);",
                             "return x > 0.0 ? x : exp(x) - 1.0;"),
    "gqa_tiling_map": ("const int b = bh / H, h = bh % H, g = h / nrep;\n"
                       "        const double *qh = q + (size_t)(b * H + h) * N * D;\n"
                       "        const double *kh = k + (size_t)(b * Hkv + g) * N * D;\n"
                       "        const double *vh = v + (size_t)(b * Hkv + g) * N * D;\n"
                       "        double *oh = out + (size_t)(b * H + h) * N * D;\n"
                       "        double *S = calloc",
                       "const int b = bh / H, h = bh % H, g = (h % Hkv) + 0 * nrep;\n"
                       "        const double *qh = q + (size_t)(b * H + h) * N * D;\n"
                       "        const double *kh = k + (size_t)(b * Hkv + g) * N * D;\n"
                       "        const double *vh = v + (size_t)(b * Hkv + g) * N * D;\n"
                       "        double *oh = out + (size_t)(b * H + h) * N * D;\n"
                       "        double *S = calloc"),
    "dq_sign_flip": ("tmp[f] = acc - c[i] * z[f];", "tmp[f] = acc + c[i] * z[f];"),
    "cos_sin_swapped_in_chain": ("cw ? cw[t] * dPhi[d] + sw[t] * dPhi[D + d]",
                                 "cw ? sw[t] * dPhi[d] + cw[t] * dPhi[D + d]"),
    "causal_exclusive_diagonal": (
        "            for (int i = 0; i < N; ++i) {\n                if (causal) {\n"
        "                    features(phi, kh + (size_t)i * D, D, cw, sw, i, kf);\n"
        "                    rank1(S, z, kf, vh + (size_t)i * D, F, D);\n                }\n"
        "                features(phi, qh + (size_t)i * D, D, cw, sw, i, qf);",
        "            for (int i = 0; i < N; ++i) {\n                if (causal && i > 0) {\n"
        "                    features(phi, kh + (size_t)(i - 1) * D, D, cw, sw, i - 1, kf);\n"
        "                    rank1(S, z, kf, vh + (size_t)(i - 1) * D, F, D);\n                }\n"
        "                features(phi, qh + (size_t)i * D, D, cw, sw, i, qf);"),
    "dv_uses_q_features": ("for (int d = 0; d < D; ++d) dvj[d] += row[d] * kf[f];",
                           "for (int d = 0; d < D; ++d) dvj[d] += row[d] * qf[(size_t)j * F + f];"),
}


def _rel(a, b):
    den = np.max(np.abs(b))
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / (den if den > 0 else 1.0))


def pins_pass(orc):
    """Run a compact set of independent pins against oracle object ``orc``."""
    with open(GOLDEN) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        q, k, v = (np.array(case[n])[None, None] for n in ("q", "k", "v"))
        cw = np.array(case["cos"]) if "cos" in case else None
        sw = np.array(case["sin"]) if "sin" in case else None
        out = orc.fwd(q, k, v, case["causal"], case["phi"], case["eps"], cw, sw)
        if not np.allclose(out, np.array(case["out"])[None, None], rtol=1e-12, atol=1e-12):
            return False
    for case in gold["grad_cases"]:
        q, k, v, g = (np.array(case[n])[None, None] for n in ("q", "k", "v", "grad_out"))
        got = orc.bwd(q, k, v, g, case["causal"], case["phi"], case["eps"])
        for a, n in zip(got, ("dq", "dk", "dv")):
            if not np.allclose(a, np.array(case[n])[None, None], rtol=1e-12, atol=1e-12):
                return False
    B, H, Hkv, N, D = 1, 4, 2, 12, 3
    x = {n: a.astype(np.float64) for n, a in draw(B, H, Hkv, N, D, 1.0, 5).items()}
    c, s = cos_sin(N)
    for causal in (True, False):
        for cw, sw in ((None, None), (c.astype(np.float64), s.astype(np.float64))):
            kw = dict(is_causal=causal, phi="elu+1", eps=1e-6, cos_weight=cw, sin_weight=sw)
            if _rel(orc.fwd(x["q"], x["k"], x["v"], **kw),
                    brute.out_np(x["q"], x["k"], x["v"], **kw)) > 1e-12:
                return False
            got = orc.bwd(x["q"], x["k"], x["v"], x["grad_out"], **kw)
            want = brute.torch_grads(x["q"], x["k"], x["v"], x["grad_out"], **kw)
            if any(_rel(a, b) > 1e-11 for a, b in zip(got, want)):
                return False
    return True


def test_unmutated_oracle_passes_pins():
    assert pins_pass(oracle.load())


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    so = oracle.build(force=True, src=str(mutated), out=str(tmp_path / "libmutant.so"))
    assert not pins_pass(oracle.load(so)), name
