"""Oracle pins: acceptance estimator (Eq. 1), survivals and chain selection.

Pinned to values the Hybrid Spark page prints (fixtures under tests/golden)
and to closed forms; none of these tests re-derives the oracle's formula.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from workloads import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def only(**kw):
    e = synth.Estimator(beta=np.zeros(15, np.float32))
    for k, v in kw.items():
        setattr(e, k, v)
    return e


def test_shared_intercept_acceptance():
    g = gold("estimator_pins.json")["shared_intercept"]
    e = only(beta=np.full(15, g["beta"], np.float32))
    h = O.estimate(e, n=5, a=0, m=0, length=15)
    assert np.allclose(h, g["acceptance"], atol=g["tol"])
    # survival still decays with position (Appendix E): S_k = h^k
    S = O.survival(h)
    assert np.all(np.diff(S) < 0)
    assert S[14] == pytest.approx(float(h[0]) ** 15, rel=1e-12)


def test_per_position_intercepts():
    g = gold("estimator_pins.json")["per_position_intercepts"]
    e = only(beta=np.array(g["beta"], np.float32))
    h = O.estimate(e, n=5, a=0, m=0, length=15)
    assert h[0] == pytest.approx(g["first_acceptance"], abs=g["tol"])
    assert h[14] == pytest.approx(g["last_acceptance"], abs=g["tol"])


def test_copy_term_scale_and_cap():
    g = gold("estimator_pins.json")["copy_term"]
    e = only(k_first=g["kappa_first"])
    # at n = 15 and m = 256 the copy term at position 1 is kappa_first ln(256/15), about 5.7
    assert O.estimate_logit(e, 1, 15, 0, g["m"]) == pytest.approx(g["logit_increase"], abs=g["tol"])
    # the copy length is capped at 256 ...
    assert O.estimate_logit(e, 1, 15, 0, 1000) == pytest.approx(O.estimate_logit(e, 1, 15, 0, 256), abs=1e-12)
    # ... a 15-token copy adds nothing, and the term is absent below a full match
    assert O.estimate_logit(e, 1, 15, 0, 15) == pytest.approx(0.0, abs=1e-12)
    assert O.estimate_logit(e, 1, 14, 0, 0) == pytest.approx(0.0, abs=1e-12)
    # the term belongs to the first position's coefficient only
    assert O.estimate_logit(e, 2, 15, 0, 256) == pytest.approx(0.0, abs=1e-12)


def test_table5_hand_values():
    g = gold("estimator_pins.json")
    t5 = g["table5_qwen3_4b"]
    e = synth.estimator_qwen3_4b()
    # the generator's transcription of Table 5 equals the fixture
    assert np.allclose(e.beta, np.array(t5["beta"], np.float32))
    for k in ("w_first", "w_rest", "delta", "l_first", "l_rest", "k_first", "k_rest"):
        assert float(getattr(e, k)) == pytest.approx(t5[k], abs=1e-6)
    hv = g["table5_hand_values"]
    for c in hv["cases"]:
        z = O.estimate_logit(e, c["k"], c["n"], c["a"], c["m"])
        assert z == pytest.approx(c["logit"], abs=hv["tol_logit"]), c
        h = O.estimate(e, c["n"], c["a"], c["m"], c["k"])[c["k"] - 1]
        assert h == pytest.approx(c["h"], abs=hv["tol_h"]), c


def test_match_length_and_agreement_terms():
    e = only(w_first=0.4, w_rest=0.1, delta=1.25)
    assert O.estimate_logit(e, 1, 9, 0, 0) == pytest.approx(0.4 * 4, abs=1e-6)
    assert O.estimate_logit(e, 3, 9, 0, 0) == pytest.approx(0.1 * 4, abs=1e-6)
    assert O.estimate_logit(e, 3, 9, 1, 0) - O.estimate_logit(e, 3, 9, 0, 0) == pytest.approx(1.25, abs=1e-6)


def test_linear_length_workload_estimator():
    # the batch-allocation workload's calibrated acceptance sigmoid(0.4 n - 1)
    e = synth.estimator_linear_length()
    for n in range(5, 16):
        h = O.estimate(e, n, 1, 0 if n < 15 else 40, 15)
        assert np.allclose(h, 1 / (1 + math.exp(-(0.4 * n - 1))), atol=1e-6)


# ---------------------------------------------------------------------------
# chain selection
# ---------------------------------------------------------------------------

def linear(first, step, n):
    return np.array([first - i * step for i in range(n)])


def chains_table8():
    """Survivals with Table 8's aggregates: the n-gram chain has 9 slots above
    lambda summing to 4.35 and 6 below summing to 1.52; DSpark has 7 slots
    summing to 5.58, all above lambda."""
    g = gold("chain_value_table8.json")
    above = linear(0.62, (9 * 0.62 - g["ngram"]["sum_above"]) / 36, 9)
    below = linear(0.29, (6 * 0.29 - g["ngram"]["below_sum"]) / 15, 6)
    Sg = np.concatenate([above, below])
    Sd = linear(0.95, (7 * 0.95 - g["dspark"]["sum_above"]) / 21, 7)
    h = Sg / np.concatenate([[1.0], Sg[:-1]])
    c = Sd / np.concatenate([[1.0], Sd[:-1]])
    return g, Sg, Sd, h, c


def test_table8_value_rule():
    g, Sg, Sd, h, c = chains_table8()
    lam = g["lambda"]
    assert Sg.sum() == pytest.approx(g["ngram"]["sum_S"], abs=1e-9)
    assert int((Sg > lam).sum()) == g["ngram"]["slots_above"]
    assert O.chain_value(Sg, lam) == pytest.approx(g["ngram"]["V"], abs=g["tol"])
    assert O.chain_value(Sd, lam) == pytest.approx(g["dspark"]["V"], abs=g["tol"])
    d = np.arange(100, 107, dtype=np.int32)
    ng = np.arange(200, 215, dtype=np.int32)
    sel = O.select(d, c, ng, h, lam, "proposed")
    assert sel["src"] == 0 and sel["len"] == 7            # the value keeps DSpark's chain
    assert np.array_equal(sel["tokens"][:7], d)
    assert np.allclose(sel["S"][:7], Sd)
    # ... although expected accepted tokens (sum S) prefer the n-gram chain
    assert Sg.sum() > Sd.sum()
    sel0 = O.select(d, c, ng, h, 0.0, "proposed")         # at price 0, V = sum S
    assert sel0["src"] == 1 and sel0["len"] == 15


def test_value_tie_goes_to_ngram():
    S = np.array([0.9, 0.8, 0.7])
    a = S / np.concatenate([[1.0], S[:-1]])
    sel = O.select(np.array([1, 2, 3], np.int32), a, np.array([4, 5, 6], np.int32), a, 0.3, "proposed")
    assert sel["src"] == 1 and sel["near"]


def test_contains_rule_merges_survivals():
    d = np.array([5, 6, 7], np.int32)
    g = np.array([5, 6, 7, 8, 9], np.int32)
    c = np.array([0.9, 0.9, 0.9])
    h = np.array([0.5, 0.99, 0.99, 0.9, 0.8])
    sel = O.select(d, c, g, h, 0.3, "proposed", K=3)
    assert sel["src"] == 2 and sel["len"] == 5
    Sd, Sg = np.cumprod(c), np.cumprod(h)
    exp = list(np.maximum(Sd, Sg[:3]))
    exp += [exp[-1] * h[3], exp[-1] * h[3] * h[4]]
    assert np.allclose(sel["S"][:5], exp, rtol=1e-12)
    assert np.all(sel["flags"][:5] == O.SLOT_POINT_MASS | O.SLOT_FROM_NGRAM)
    # not a prefix (or not longer) -> no merge
    assert O.select(d, c, np.array([5, 6, 1, 8], np.int32), h[:4], 0.3, "proposed", K=3)["src"] != 2
    assert O.select(d, c, np.array([5, 6, 7], np.int32), h[:3], 0.3, "proposed", K=3)["src"] != 2


def test_policies():
    d = np.array([5, 6, 7], np.int32)
    c = np.array([0.95, 0.95, 0.95])
    g = np.array([5, 6, 7, 8, 9], np.int32)
    h = np.array([0.2, 0.9, 0.9, 0.9, 0.9])
    ext = O.select(d, c, g, h, 0.3, "extension", model_point_mass=False, K=3)
    assert ext["src"] == 3 and ext["len"] == 5
    assert list(ext["flags"][:5]) == [0, 0, 0, 3, 3]      # model slots probabilistic, tail point masses
    Sd = np.cumprod(c)
    assert np.allclose(ext["S"][:5], [*Sd, Sd[-1] * 0.9, Sd[-1] * 0.81], rtol=1e-12)
    g2 = np.array([1, 2], np.int32)
    assert O.select(d, c, g2, h[:2], 0.3, "ngram_first")["src"] == 1
    assert O.select(d, c, g2[:0], h[:0], 0.3, "ngram_first")["src"] == 0
    assert O.select(d, c, g2, h[:2], 0.3, "extension")["src"] == 0
    assert O.select(d, c, g2, h[:2], 0.3, "model_only")["src"] == 0
    assert O.select(d, c, g2, h[:2], 0.3, "ngram_only")["len"] == 2
    # greedy drafting: model slots are point masses
    assert np.all(O.select(d, c, g2[:0], h[:0], 0.3, "proposed", model_point_mass=True)["flags"][:3] == 1)
