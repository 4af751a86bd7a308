"""The library's host budget sizing (spec_size_budget) against the oracle: the
same budget, slot price and goodput curve, bit for bit, on random survivals,
with and without the eager step of Eq. (4), and on the survivals the batch
allocation produces for the BS 128 workload.  Host code only: no GPU."""
import numpy as np
import pytest

from oracle import oracle as O


@pytest.fixture(scope="module")
def S():
    import draft_verification_spec_amd as S
    return S


@pytest.mark.parametrize("seed", range(30))
def test_matches_oracle_random(S, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 5000))
    surv = (rng.random(n) ** rng.uniform(0.2, 4)).astype(np.float32)
    surv[rng.random(n) < 0.1] = 0.0
    B = int(rng.integers(1, 300))
    c0, p = rng.uniform(0.1, 100), rng.uniform(0, 2)
    b_max = int(rng.integers(0, n + 10)) if rng.random() < 0.5 else 0
    kw = {}
    if rng.random() < 0.5 and n > 0:
        limit = B + int(rng.integers(0, n))
        kw = dict(graph_limit=limit, n_tokens=B,
                  eager=c0 + p * np.arange(limit + 1, limit + 1 + n) + rng.uniform(0, 5, n))
    b, lam, g, curve = S.spec_size_budget(surv, B, c0, p, b_max=b_max, curve=True, **kw)
    ob, olam, oG = O.size_budget(surv, B, c0, p, b_max=b_max if b_max > 0 else None, **kw)
    assert b == ob and lam == olam and g == oG[ob]
    assert np.array_equal(curve, oG)


def test_all_zero_and_empty(S):
    assert S.spec_size_budget(np.zeros(0, np.float32), 4, 2.0, 0.5) == (0, 1.0, 2.0)
    b, lam, g = S.spec_size_budget(np.zeros(100, np.float32), 4, 2.0, 0.5)
    assert b == 0 and lam == 1.0


def test_rejects_bad_cost(S):
    import draft_verification_spec_amd._lib as L
    with pytest.raises(Exception):
        S.spec_size_budget(np.ones(4, np.float32), 4, 0.0, 0.5)
    with pytest.raises(Exception):
        S.spec_size_budget(np.ones(4, np.float32), 4, 1.0, -0.5)


def test_budget_workload_survivals(S):
    """Survivals of the chosen chains of the BS 128 batch-allocation workload
    (the oracle's selection), sized at the pages' BS-128 slot price scale."""
    from workloads import synth
    c = synth.config2()
    d, dl, f = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], 15, 256)
    al = O.allocate_budget(c["model_tokens"], c["model_conf_logit"], True, c["model_point_mass"], d, dl, f,
                           c["estimator"], c["lam"], c["budget"])
    surv = al["S"].astype(np.float32).ravel()
    sizes = []
    for c0, p in ((128.0, 0.3), (128.0, 1.0), (50.0, 0.05)):
        b, lam, g = S.spec_size_budget(surv, c["BS"], c0, p)
        ob, olam, oG = O.size_budget(surv, c["BS"], c0, p)
        assert (b, lam) == (ob, olam) and g == oG[ob]
        sizes.append(b)
    # a slot costing as much as a whole request's step is never worth it;
    # cheaper slots buy most of the batch's chains
    assert sizes[1] == 0 and 0 < sizes[0] < sizes[2] <= (surv > 0).sum()
