"""Oracle pins: losslessness of the chain-selection policies at the level of
the whole step (Hybrid Spark, Section 4.5 and Appendix H, Table 9).

A tiny Markov target and a tiny Markov drafter over three tokens; each round,
for every trial, the drafter proposes a 2-token chain (sampled from q, or its
argmax when drafting is greedy) with confidences, where the second confidence
depends on the token sampled first (the drafter is confident after token 0,
as a confidence head that reads its own sample); a model-free n-gram chain is
a fixed function of the last context token (absent after token 1).  The
oracle's selection (each policy), its batch allocation under a budget that
cuts slots, and its rejection-sampling verification then emit the round's
tokens.  The law of the first three emitted tokens is compared with the
target's exact law by chi-square.

Table 9 (tests/golden/losslessness_table9.json) says which combinations keep
the target's law: every policy at T = 0 and with greedy drafting; with
probabilistic drafting at T > 0, n-gram-first and extension but not the
proposed policy.  The 'no' entry must show a clear bias, the 'yes' entries
none.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE9 = json.load(open(os.path.join(HERE, "golden", "losslessness_table9.json")))

V, K, L, X0, LENGTH = 3, 2, 3, 2, 3
ZP = np.array([[0.2, 1.1, -0.4], [0.9, -0.3, 0.5], [-0.2, 0.1, -0.2]])   # target logits, row = previous token
ZQ = np.array([[0.6, 0.4, -0.9], [0.3, 0.2, 0.1], [0.7, 0.2, -0.3]])    # drafter logits
NGRAM = {0: [1, 2, 0], 1: [], 2: [0, 1, 1]}                              # model-free chain after each token
H = 0.6                                                                  # its per-slot estimate
LAM = 0.3


def confidences(y1):
    """Second confidence read from the first sampled token."""
    return np.array([0.5, 0.95 if y1 == 0 else 0.05])


def run_policy(policy, drafting, T, N, seed):
    rng = np.random.Generator(np.random.Philox(seed))
    Pq = scipy.special.softmax(ZQ / (T if T > 0 else 1.0), axis=1)
    seqs = np.full((N, LENGTH), -1, np.int64)
    filled = np.zeros(N, np.int64)
    last = np.full(N, X0, np.int64)
    while (filled < LENGTH).any():
        act = np.nonzero(filled < LENGTH)[0]
        n = len(act)
        toks = np.full((n, L), -1, np.int32)
        flags = np.zeros((n, L), np.uint8)
        S = np.zeros((n, L))
        lens = np.zeros(n, np.int32)
        for i, a in enumerate(act):
            x = int(last[a])
            if drafting == "greedy":
                y1 = int(np.argmax(Pq[x]))
                y2 = int(np.argmax(Pq[y1]))
            else:
                y1 = int(rng.choice(V, p=Pq[x]))
                y2 = int(rng.choice(V, p=Pq[y1]))
            g = NGRAM[x]
            sel = O.select(np.array([y1, y2]), confidences(y1), np.array(g, np.int32), np.full(len(g), H), LAM,
                           policy, model_point_mass=drafting == "greedy", K=K, ld=L)
            toks[i], flags[i], S[i], lens[i] = sel["tokens"], sel["flags"], sel["S"], sel["len"]
        alloc, _, _, _ = O.allocate(lens, S, 2 * n)
        # Markov rows: slot k is scored by the row of the token before it
        prev = np.concatenate([last[act][:, None], np.where(toks >= 0, toks, 0)], axis=1)   # [n, L + 1]
        tgt = ZP[prev].astype(np.float32).reshape(-1, V)
        dft = ZQ[prev[:, :L]].astype(np.float32).reshape(-1, V)
        res = O.verify_chain(tgt, np.arange(n) * (L + 1), toks, flags, alloc,
                             rng.random((n, L), dtype=np.float32), rng.random(n, dtype=np.float32), T,
                             draft_logits=dft, draft_row_base=np.arange(n) * L)
        out, num = res["out_tokens"], res["out_num"]
        for k in range(L + 1):
            m = (num > k) & (filled[act] < LENGTH)
            idx = act[m]
            seqs[idx, filled[idx]] = out[m, k]
            filled[idx] += 1
            last[idx] = out[m, k]
    return seqs


def target_law(T):
    P = scipy.special.softmax(ZP / T, axis=1)
    law = np.zeros((V,) * LENGTH)
    for cell in np.ndindex(*law.shape):
        pr, prev = 1.0, X0
        for t in cell:
            pr *= P[prev, t]
            prev = t
        law[cell] = pr
    return law.ravel()


def chi2_p(seqs, law):
    idx = np.zeros(len(seqs), np.int64)
    for t in range(LENGTH):
        idx = idx * V + seqs[:, t]
    obs = np.bincount(idx, minlength=V ** LENGTH)
    return scipy.stats.chisquare(obs, law * len(seqs)).pvalue


def greedy_decode():
    seq, prev = [], X0
    for _ in range(LENGTH):
        prev = int(np.argmax(ZP[prev]))
        seq.append(prev)
    return seq


CASES = [(row["T"], row["drafting"], pol, row[pol]) for row in TABLE9["rows"]
         for pol in ("proposed", "ngram_first", "extension")]


@pytest.mark.parametrize("T_row,drafting,policy,lossless", CASES)
def test_table9_policy_losslessness(T_row, drafting, policy, lossless):
    if T_row == "0":
        # T = 0: the output is the target's greedy decode whatever the drafts
        for d in ("greedy", "probabilistic"):
            seqs = run_policy(policy, d, 0.0, 3000, 9)
            assert np.all(seqs == np.array(greedy_decode())), (policy, d)
        return
    T = 1.0
    seqs = run_policy(policy, drafting, T, 40000, 11 + len(policy) + len(drafting))
    p = chi2_p(seqs, target_law(T))
    print(f"T {T_row} {drafting} {policy}: chi-square p = {p:.3g}")
    if lossless:
        assert p > 1e-4, (policy, drafting, p)
    else:
        assert p < 1e-12, (policy, drafting, p)


def test_every_policy_path_is_exercised():
    """The Monte Carlo reaches each selection outcome it is meant to test:
    the proposed policy keeps the drafter's chain after token 0 and the
    n-gram chain otherwise; the contains rule merges; extension appends a
    tail; n-gram-first falls back to the drafter without a match."""
    seen = set()
    for y1 in range(V):
        for y2 in range(V):
            for x in range(V):
                g = NGRAM[x]
                for pol in ("proposed", "ngram_first", "extension"):
                    sel = O.select(np.array([y1, y2]), confidences(y1), np.array(g, np.int32), np.full(len(g), H),
                                   LAM, pol, model_point_mass=False, K=K, ld=L)
                    seen.add((pol, sel["src"]))
    assert {("proposed", 0), ("proposed", 1), ("proposed", 2), ("ngram_first", 0), ("ngram_first", 1),
            ("extension", 0), ("extension", 3)} <= seen


@pytest.mark.parametrize("mutation,policy", [(3, "extension"), (4, "ngram_first")])
def test_policy_monte_carlo_detects_planted_mistake(tmp_path, mutation, policy):
    """The same Monte Carlo rejects two plausible policy mistakes compiled
    into the oracle: extension tail slots verified against q instead of as
    point masses, and an n-gram-first choice that reads the drafter's first
    sample."""
    path = O.build_mutant(str(tmp_path / f"liboracle_m{mutation}.so"), mutation)
    with O.using_library(path):
        seqs = run_policy(policy, "probabilistic", 1.0, 40000, 77)
    assert chi2_p(seqs, target_law(1.0)) < 1e-8
