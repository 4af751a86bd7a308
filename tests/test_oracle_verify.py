"""Oracle pins: chain verification by rejection sampling and commit.

* Monte Carlo losslessness: speculative rounds over a tiny Markov target must
  reproduce the target's law on whole sequences (chi-square), for
  probabilistic, point-mass and mixed drafts, at T = 1 and T = 0.7 -- and the
  same test must reject two planted mistakes compiled into the oracle.
* Acceptance-rate closed forms (Hybrid Spark, Section 5.8): a greedy draft x
  is accepted with p(x); a sampled draft with sum_x min(p(x), q(x)).
* T = 0 gives plain greedy decoding; q = p always accepts; the prefix
  advances by r + 1; probabilities equal a library softmax.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import oracle as O
from workloads import synth


def softmax_rows(Z, T):
    return scipy.special.softmax(np.asarray(Z, np.float64) / T, axis=-1)


def sample_rows(rng, P):
    u = rng.random(P.shape[0])
    cdf = np.cumsum(P, axis=1)
    return np.minimum((u[:, None] >= cdf).sum(1), P.shape[1] - 1)


def speculative_sequences(Zp, Zq, T, B, pm_slots, N, length, seed, x0=0):
    """Run speculative rounds until every trial has ``length`` tokens."""
    rng = np.random.Generator(np.random.Philox(seed))
    V = Zp.shape[0]
    Pq = softmax_rows(Zq, T)
    seqs = np.full((N, length), -1, np.int64)
    filled = np.zeros(N, np.int64)
    last = np.full(N, x0, np.int64)
    flags = np.array([O.SLOT_POINT_MASS if pm else 0 for pm in pm_slots], np.uint8)
    while (filled < length).any():
        act = np.nonzero(filled < length)[0]
        n = len(act)
        y = np.zeros((n, B), np.int64)
        prev = last[act]
        for i in range(B):
            y[:, i] = np.argmax(Zq[prev], axis=1) if pm_slots[i] else sample_rows(rng, Pq[prev])
            prev = y[:, i]
        toks = np.concatenate([last[act][:, None], y], axis=1)
        tgt = Zp[toks].astype(np.float32).reshape(-1, V)
        dft = Zq[toks[:, :B]].astype(np.float32).reshape(-1, V)
        res = O.verify_chain(tgt, np.arange(n) * (B + 1), y.astype(np.int32), np.tile(flags, (n, 1)),
                             np.full(n, B, np.int32), rng.random((n, B), dtype=np.float32),
                             rng.random(n, dtype=np.float32), T,
                             draft_logits=dft, draft_row_base=np.arange(n) * B)
        out, num = res["out_tokens"], res["out_num"]
        assert np.all(num == res["out_accepted"] + 1)
        for k in range(B + 1):
            m = (num > k) & (filled[act] < length)
            idx = act[m]
            seqs[idx, filled[idx]] = out[m, k]
            filled[idx] += 1
            last[idx] = out[m, k]
    return seqs


def target_law(Zp, T, length, x0=0):
    V = Zp.shape[0]
    P = softmax_rows(Zp, T)
    law = np.zeros((V,) * length)
    for cell in np.ndindex(*law.shape):
        pr, prev = 1.0, x0
        for t in cell:
            pr *= P[prev, t]
            prev = t
        law[cell] = pr
    return law.ravel()


def chi2_pvalue(seqs, law, V):
    idx = np.zeros(len(seqs), np.int64)
    for t in range(seqs.shape[1]):
        idx = idx * V + seqs[:, t]
    obs = np.bincount(idx, minlength=V ** seqs.shape[1]).astype(np.float64)
    exp = law * len(seqs)
    keep = exp >= 5
    obs2 = np.append(obs[keep], obs[~keep].sum())
    exp2 = np.append(exp[keep], exp[~keep].sum())
    if exp2[-1] == 0:
        obs2, exp2 = obs2[:-1], exp2[:-1]
    return scipy.stats.chisquare(obs2, exp2 * obs2.sum() / exp2.sum()).pvalue


def markov(V, seed, scale=1.5):
    rng = np.random.Generator(np.random.Philox(seed))
    Zp = rng.standard_normal((V, V)) * scale
    Zq = Zp + rng.standard_normal((V, V)) * scale   # a poor drafter
    return Zp, Zq


CASES = [  # (V, B, T, point-mass pattern)
    (4, 3, 1.0, (0, 0, 0)),
    (4, 3, 0.7, (1, 1, 1)),
    (4, 3, 1.0, (0, 1, 0)),
    (2, 1, 0.7, (0,)),
    (8, 2, 1.0, (1, 0)),
]


@pytest.mark.parametrize("V,B,T,pm", CASES)
def test_losslessness_monte_carlo(V, B, T, pm):
    Zp, Zq = markov(V, 100 + V + B)
    length = 4 if V <= 4 else 3
    seqs = speculative_sequences(Zp, Zq, T, B, pm, N=300_000, length=length, seed=5 + V * 10 + B)
    p = chi2_pvalue(seqs, target_law(Zp, T, length), V)
    assert p > 1e-4, p


@pytest.mark.parametrize("mutation", [1, 2])
def test_monte_carlo_detects_planted_mistake(tmp_path, mutation):
    path = O.build_mutant(str(tmp_path / f"liboracle_m{mutation}.so"), mutation)
    Zp, Zq = markov(4, 107)
    with O.using_library(path):
        seqs = speculative_sequences(Zp, Zq, 1.0, 3, (0, 0, 0), N=300_000, length=4, seed=9)
    assert chi2_pvalue(seqs, target_law(Zp, 1.0, 4), 4) < 1e-8


@pytest.mark.parametrize("pm", [0, 1])
def test_acceptance_rate_closed_forms(pm):
    rng = np.random.Generator(np.random.Philox(21))
    V, N, T = 8, 200_000, 1.0
    z = rng.standard_normal(V) * 1.5
    w = z + rng.standard_normal(V)
    p, q = softmax_rows(z, T), softmax_rows(w, T)
    if pm:
        y = np.full(N, int(np.argmax(w)))
        expect = p[int(np.argmax(w))]
    else:
        y = sample_rows(rng, np.tile(q, (N, 1)))
        expect = np.minimum(p, q).sum()
    tgt = np.tile(np.stack([z, z]).astype(np.float32), (N, 1))
    res = O.verify_chain(tgt, np.arange(N) * 2, y[:, None].astype(np.int32), np.full((N, 1), pm, np.uint8),
                         np.ones(N, np.int32), rng.random((N, 1), dtype=np.float32),
                         rng.random(N, dtype=np.float32), T,
                         draft_logits=np.tile(w.astype(np.float32), (N, 1)), draft_row_base=np.arange(N))
    rate = res["out_accepted"].mean()
    assert abs(rate - expect) < 5 * np.sqrt(expect * (1 - expect) / N)


def test_greedy_at_temperature_zero_and_probabilities():
    c = synth.config0(BS=6, V=3001)
    B = c["B"]
    z = c["target"].reshape(-1, c["V"])
    res = O.verify_chain(z, np.arange(6) * (B + 1), c["tokens"], np.zeros((6, B), np.uint8),
                         np.full(6, B, np.int32), c["u_acc"], c["u_smp"], 0.0,
                         draft_logits=c["draft"].reshape(-1, c["V"]), draft_row_base=np.arange(6) * B)
    am = np.argmax(c["target"], axis=-1)
    for r in range(6):
        n = 0
        while n < B and c["tokens"][r, n] == am[r, n]:
            n += 1
        assert res["out_accepted"][r] == n and res["out_num"][r] == n + 1
        assert list(res["out_tokens"][r, :n]) == list(c["tokens"][r, :n])
        assert res["out_tokens"][r, n] == am[r, n]
    # T > 0: slot probabilities equal a library softmax, q likewise
    T = 0.8
    res = O.verify_chain(z, np.arange(6) * (B + 1), c["tokens"], np.zeros((6, B), np.uint8),
                         np.full(6, B, np.int32), c["u_acc"], c["u_smp"], T,
                         draft_logits=c["draft"].reshape(-1, c["V"]), draft_row_base=np.arange(6) * B)
    P = softmax_rows(c["target"][:, :B], T)
    Q = softmax_rows(c["draft"], T)
    for r in range(6):
        for i in range(B):
            y = c["tokens"][r, i]
            assert res["out_p"][r, i] == pytest.approx(P[r, i, y], rel=1e-12)
            assert res["out_q"][r, i] == pytest.approx(Q[r, i, y], rel=1e-12)
        a = res["out_accepted"][r]
        assert res["out_num"][r] == a + 1
        assert list(res["out_tokens"][r, :a]) == list(c["tokens"][r, :a])
        for i in range(a):   # every accepted slot passed u < p/q
            assert c["u_acc"][r, i] < P[r, i, c["tokens"][r, i]] / Q[r, i, c["tokens"][r, i]]
        if a < B:
            assert not c["u_acc"][r, a] < P[r, a, c["tokens"][r, a]] / Q[r, a, c["tokens"][r, a]]


def test_identical_draft_always_accepted_and_bonus():
    rng = np.random.Generator(np.random.Philox(4))
    V, B, n = 50, 5, 500
    z = rng.standard_normal((n, B + 1, V)).astype(np.float32)
    y = np.stack([sample_rows(rng, softmax_rows(z[:, i], 1.0)) for i in range(B)], 1).astype(np.int32)
    res = O.verify_chain(z.reshape(-1, V), np.arange(n) * (B + 1), y, np.zeros((n, B), np.uint8),
                         np.full(n, B, np.int32), rng.random((n, B), dtype=np.float32),
                         rng.random(n, dtype=np.float32), 1.0,
                         draft_logits=z[:, :B].reshape(-1, V).copy(), draft_row_base=np.arange(n) * B)
    assert np.all(res["out_accepted"] == B) and np.all(res["out_num"] == B + 1)
    # the bonus is a draw from p_{B+1}: its empirical law tracks the row's mass
    assert np.all((res["out_tokens"][:, B] >= 0) & (res["out_tokens"][:, B] < V))


def test_bf16_input_equals_upcast():
    c = synth.config0(BS=3, V=2000)
    bits = synth.f32_to_bf16_bits(c["target"])
    up = synth.bf16_bits_to_f32(bits)
    args = (np.arange(3) * 8, c["tokens"], np.full((3, 7), 1, np.uint8), np.full(3, 7, np.int32),
            c["u_acc"], c["u_smp"], 1.0)
    a = O.verify_chain(bits.reshape(-1, 2000), *args)
    b = O.verify_chain(up.reshape(-1, 2000), *args)
    for k in ("out_tokens", "out_num", "out_p"):
        assert np.array_equal(a[k], b[k])


def test_edge_cases_zero_slots_bad_token_commit():
    rng = np.random.Generator(np.random.Philox(8))
    V = 100
    z = rng.standard_normal((2 * 3, V)).astype(np.float32)
    toks = np.array([[5, 6], [V + 3, 1]], np.int32)
    res = O.verify_chain(z, np.array([0, 3]), toks, np.ones((2, 2), np.uint8), np.array([0, 2], np.int32),
                         rng.random((2, 2), dtype=np.float32), rng.random(2, dtype=np.float32), 0.0)
    assert res["out_num"][0] == 1 and res["out_tokens"][0, 0] == np.argmax(z[0])
    assert res["flags"][1] & O.BAD_TOKEN and res["out_accepted"][1] == 0
    assert res["out_tokens"][1, 0] == np.argmax(z[3])
    ctx = np.zeros((2, 6), np.int32)
    ctx_len = np.array([2, 5], np.int32)
    fl = np.zeros(2, np.uint32)
    out = np.array([[7, 8, -1], [9, -1, -1]], np.int32)
    ctx2, len2 = O.commit(ctx, ctx_len, 6, out, np.array([2, 2], np.int32), fl)
    assert list(len2) == [4, 5] and list(ctx2[0, 2:4]) == [7, 8]
    assert fl[1] & O.CTX_OVERFLOW and not fl[0] & O.CTX_OVERFLOW


def _draw_windows(z, u, T, seed):
    """Bonus draws (no slots) from rows z [n, V] with uniforms u [n]."""
    n, V = z.shape
    res = O.verify_chain(z.astype(np.float32), np.arange(n), np.zeros((n, 1), np.int32), np.ones((n, 1), np.uint8),
                         np.zeros(n, np.int32), np.zeros((n, 1), np.float32), u.astype(np.float32), T)
    return res


def test_tie_window_holds_every_nearby_draw():
    """The draw's tie window (the tokens whose CDF interval meets the band of
    1e-6 W around u'W) is one token away from near ties and, at a near tie,
    holds the token picked by every inverse-CDF draw whose running sums
    differ from the oracle's by less than the band: here float32 running
    sums, sums in reversed chunk order and weights perturbed by 1e-9."""
    rng = np.random.Generator(np.random.Philox(41))
    n, V, T = 400, 40, 1.0
    z = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    P = softmax_rows(z, T)
    cdf = np.cumsum(P, axis=1)
    # half the uniforms sit on a CDF boundary (to fp32 precision), half anywhere
    k = rng.integers(1, V - 1, n)
    u = np.where(np.arange(n) % 2 == 0, cdf[np.arange(n), k - 1] / cdf[:, -1], rng.random(n)).astype(np.float32)
    res = _draw_windows(z, u, T, 41)
    tok, lo, hi = res["out_tokens"][:, 0], res["win_lo"], res["win_hi"]
    near = (res["flags"] & O.SAMPLE_NEAR) != 0
    assert near[0::2].mean() > 0.9                       # boundary uniforms are near ties
    assert np.all(lo <= tok) and np.all(tok <= hi)
    assert np.array_equal(lo[~near], tok[~near]) and np.array_equal(hi[~near], tok[~near])
    assert np.all(hi[near] > lo[near])                   # a boundary window spans both sides
    for r in range(n):
        t = float(u[r])
        picks = []
        w = P[r].astype(np.float32)
        picks.append(int(np.searchsorted(np.cumsum(w, dtype=np.float32), t * w.sum(dtype=np.float32), "right")))
        wr = P[r] * (1 + 1e-9 * rng.standard_normal(V))
        picks.append(int(np.searchsorted(np.cumsum(wr), t * wr.sum(), "right")))
        chunks = np.array_split(P[r], 5)
        run = np.concatenate([np.cumsum(c) + sum(x.sum() for x in chunks[:i]) for i, c in enumerate(chunks)])
        picks.append(int(np.searchsorted(run, t * sum(c.sum() for c in reversed(chunks)), "right")))
        for p in picks:
            p = min(p, V - 1)
            assert lo[r] <= p <= hi[r], (r, p, lo[r], hi[r])


def test_bonus_row_probability():
    """out_p's column b is p of the bonus row at the bonus token (a library
    softmax) when every slot passed, 1 at T = 0, and 0 after a rejection."""
    rng = np.random.Generator(np.random.Philox(42))
    n, V, B = 60, 300, 3
    z = (rng.standard_normal((n, B + 1, V)) * 2).astype(np.float32)
    y = rng.integers(0, V, (n, B)).astype(np.int32)
    y[: n // 2] = np.argmax(z[: n // 2, :B], -1)       # greedy drafts: accepted at T = 0
    u_acc = np.where(np.arange(n)[:, None] < n // 2, 0.0, rng.random((n, B))).astype(np.float32)
    u_smp = rng.random(n, dtype=np.float32)
    for T in (0.0, 0.9):
        res = O.verify_chain(z.reshape(-1, V), np.arange(n) * (B + 1), y, np.ones((n, B), np.uint8),
                             np.full(n, B, np.int32), u_acc, u_smp, T)
        P = softmax_rows(z[:, B], T) if T > 0 else None
        for r in range(n):
            a = res["out_accepted"][r]
            if a < B:
                assert res["out_p"][r, B] == 0.0
            elif T == 0:
                assert res["out_p"][r, B] == 1.0
            else:
                assert res["out_p"][r, B] == pytest.approx(P[r, res["out_tokens"][r, B]], rel=1e-12)
        assert (res["out_accepted"] == B).sum() >= n // 2
