"""Pins of the oracle's budget sizing and slot price (Hybrid Spark, Section 2
"Adaptive verification", Section 4.3 Eq. (2), Appendix F Eq. (4)) and of the
stale-sizing shortfall (Appendix O, Eq. (5) and Table 16)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(S, B, cost):
    """Best goodput over every subset of slots (the cost depends only on the
    subset's size): (best G, sizes that reach it)."""
    best, sizes = -1.0, set()
    for k in range(len(S) + 1):
        c = cost(k)
        if c <= 0:
            continue
        for sub in itertools.combinations(range(len(S)), k):
            g = (B + sum(float(np.float32(S[i])) for i in sub)) / c
            if g > best + 1e-12:
                best, sizes = g, {k}
            elif abs(g - best) <= 1e-12:
                sizes.add(k)
    return best, sizes


@pytest.mark.parametrize("seed", range(40))
def test_exhaustive_subsets_linear_cost(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    S = rng.random(n).astype(np.float32) ** rng.uniform(0.3, 3)
    B = int(rng.integers(1, 6))
    c0, p = rng.uniform(0.5, 20), rng.uniform(0.05, 2)
    b, lam, G = O.size_budget(S, B, c0, p)
    best, sizes = brute_force(S, B, lambda k: c0 + p * k)
    assert G[b] == pytest.approx(best, rel=1e-12)
    assert b == min(sizes)
    assert lam == pytest.approx(G[b] * p, rel=1e-15)


@pytest.mark.parametrize("seed", range(20))
def test_slot_pays_only_above_the_price(seed):
    """Eq. (2): with a linear cost a slot improves goodput only when its survival
    exceeds lambda = G(b*) p, so the chosen slots are exactly those above the
    price (ties at the price may go either way)."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(20, 400))
    S = (rng.random(n) ** 2).astype(np.float32)
    B, c0, p = int(rng.integers(4, 200)), rng.uniform(1, 100), rng.uniform(0.01, 1)
    b, lam, G = O.size_budget(S, B, c0, p)
    s = np.sort(S.astype(np.float64))[::-1]
    assert (s[:b] >= lam - 1e-12).all()
    assert (s[b:] <= lam + 1e-12).all()
    # and the goodput curve is unimodal: rising up to b*, then falling
    assert (np.diff(G[:b + 1]) > -1e-15).all() and (np.diff(G[b:]) < 1e-15).all()


def test_no_slot_worth_its_price():
    b, lam, G = O.size_budget(np.full(10, 0.05, np.float32), 8, 10.0, 1.0)   # G(0) = 0.8, slots add 0.05 for 1.0
    assert b == 0 and lam == pytest.approx(0.8)


def test_budget_capped_by_b_max():
    b, lam, G = O.size_budget(np.full(50, 0.99, np.float32), 4, 100.0, 0.1, b_max=12)
    assert b == 12 and len(G) == 13


@pytest.mark.parametrize("seed", range(12))
def test_eager_jump_exhaustive(seed):
    """Eq. (4): past the graph capture limit the cost is the larger of the
    linear model and the profiled eager step; the optimum over every subset
    is still found."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(2, 10))
    S = rng.random(n).astype(np.float32)
    B = int(rng.integers(1, 5))
    c0, p = rng.uniform(1, 5), rng.uniform(0.05, 0.5)
    N, limit = B, B + int(rng.integers(0, n))
    eager = c0 + p * np.arange(limit + 1, limit + 1 + n) - N + rng.uniform(0, 3, n) * (rng.random(n) < 0.7)
    eager = eager[: int(rng.integers(1, n + 1))]
    cost = lambda k: O.step_cost(k, c0, p, limit, N, eager)
    b, lam, G = O.size_budget(S, B, c0, p, graph_limit=limit, n_tokens=N, eager=eager)
    best, sizes = brute_force(S, B, cost)
    assert G[b] == pytest.approx(best, rel=1e-12) and b == min(sizes)


def test_eager_jump_stops_the_budget_at_the_limit():
    # every slot is worth 0.9 at price ~0.01, but past 4 draft tokens the step
    # runs eagerly at three times the cost
    S = np.full(16, 0.9, np.float32)
    eager = np.full(32, 3.0)
    b, lam, G = O.size_budget(S, 8, 1.0, 0.01, graph_limit=8 + 4, n_tokens=8, eager=eager)
    assert b == 4
    assert O.step_cost(4, 1.0, 0.01, 12, 8, eager) == pytest.approx(1.04)
    assert O.step_cost(5, 1.0, 0.01, 12, 8, eager) == pytest.approx(3.0)
    assert O.step_cost(40, 1.0, 0.01, 12, 8, eager) < 0   # past the profiled table


def test_eq5_reproduces_table16():
    """Appendix O, Table 16: the Pred. column is Eq. (5) of the sigma column and
    the number of requests with survivals (rounding of sigma to 0.01 and of the
    prediction to 0.01 allowed)."""
    g = json.load(open(os.path.join(GOLDEN, "stale_sizing_table16.json")))
    for row in g["rows"]:
        lo_b, hi_b = g["requests_with_survivals"][str(row["bs"])]
        lo = O.stale_shortfall(row["sigma"] - 0.005, lo_b) - 0.005
        hi = O.stale_shortfall(row["sigma"] + 0.005, hi_b) + 0.005
        assert lo <= row["pred"] <= hi, row
    # a half-normal constant or a linear growth in B would not fit
    assert abs(np.sqrt(1 / (2 * np.pi)) * 1.37 * 2 - 2.16) > 0.5
    assert abs(np.sqrt(2 / np.pi) * 1.37 * 126 - 12.24) > 100


def test_stale_sizing_simulation_follows_eq5():
    """Appendix O's methodology on synthetic batches: fresh survivals of B
    requests; the stale ones switch a request's chain (a match that appears or
    vanishes) with some probability.  The per-request miscount d has a measured
    sigma; the batch shortfall on steps where the stale budget is too small
    follows Eq. (5) (the pages find 0.77-1.14 of the prediction at BS 32 and
    128), and the goodput lost by sizing from the stale survivals is never
    negative and falls as the batch grows."""
    rng = np.random.default_rng(2026)
    c0_per_req, p = 1.0, 0.02
    losses = {}
    for B in (32, 128):
        d_all, short, lost = [], [], []
        for step in range(400):
            # a request copies (a long, confident chain) or not (a short, weak
            # one); between the stale and the fresh step its state flips with
            # probability 0.12 either way, so the miscount has mean zero
            copying = rng.random(B) < 0.5
            flip = rng.random(B) < 0.12
            strong = np.cumprod(rng.uniform(0.85, 0.99, (B, 15)), axis=1)
            weak = np.cumprod(rng.uniform(0.2, 0.6, (B, 15)), axis=1)
            fresh = np.where(copying[:, None], strong, weak)
            stale = np.where((copying ^ flip)[:, None], strong, weak)
            d = stale.sum(axis=1) - fresh.sum(axis=1)
            d_all.append(d)
            D = d.sum()
            if D < 0:
                short.append(-D)
            c0 = c0_per_req * B
            bf, lf, Gf = O.size_budget(fresh.astype(np.float32), B, c0, p)
            bs_, ls, Gs = O.size_budget(stale.astype(np.float32), B, c0, p)
            lost.append(1.0 - Gf[min(bs_, len(Gf) - 1)] / Gf[bf])
        sigma = np.concatenate(d_all).std()
        ratio = np.mean(short) / O.stale_shortfall(sigma, B)
        assert 0.75 <= ratio <= 1.25, (B, ratio)
        assert min(lost) >= -1e-12
        losses[B] = np.mean(lost)
    assert losses[128] < losses[32]
