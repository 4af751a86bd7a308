"""Property-based tests (Hypothesis) of the oracle and of the library's host
sizing: invariants that hold for every input, searched over generated cases
and shrunk to a smallest counterexample on failure.  CPU only; the search is
derandomized and keeps no example database, so every run checks the same
cases."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import oracle as O

CASES = settings(max_examples=150, deadline=None, derandomize=True, database=None)


@st.composite
def texts(draw, max_len=60, alphabet=3):
    n = draw(st.integers(1, max_len))
    return np.array(draw(st.lists(st.integers(0, alphabet - 1), min_size=n, max_size=n)), np.int32)


@CASES
@given(x=texts(), n_min=st.integers(1, 4), extra=st.integers(0, 4), cap=st.sampled_from([2, 3, 5, 256]))
def test_ngram_draft_is_an_earlier_occurrence_of_the_longest_suffix(x, n_min, extra, cap):
    """[HS] Section 4.1: the draft continues an earlier occurrence of the
    context's suffix of the reported length; no earlier position matches a
    longer suffix (up to the cap), and the draft is the text that follows."""
    n_max = n_min + extra
    cap = max(cap, n_max)
    T = len(x)
    d, dl, f = O.ngram_draft(x[None, :], np.array([T], np.int32), n_min, n_max, 15, cap)
    n, a, m, j = (int(v) for v in f[0])
    # the best match length over all earlier end positions, by direct comparison
    def match(jj):
        l = 0
        while l < min(jj + 1, cap) and x[jj - l] == x[T - 1 - l]:
            l += 1
        return l
    lens = [match(jj) for jj in range(T - 1)]
    best = max(lens, default=0)
    if best < n_min:
        assert dl[0] == 0 and n == 0 and m == 0
        return
    assert j == max(jj for jj in range(T - 1) if lens[jj] == best)   # most recent of the longest
    assert n == min(best, n_max) and (m == best if best >= n_max else m == 0)
    L = min(15, T - 1 - j)
    assert dl[0] == L and np.array_equal(d[0, :L], x[j + 1:j + 1 + L])


@st.composite
def chains(draw):
    bs = draw(st.integers(1, 6))
    ld = draw(st.integers(1, 6))
    lens = np.array(draw(st.lists(st.integers(0, ld), min_size=bs, max_size=bs)), np.int32)
    # survivals on a coarse grid (ties are common), non-increasing along a chain
    S = np.zeros((bs, ld))
    for r in range(bs):
        k = int(lens[r])
        v = sorted(draw(st.lists(st.integers(1, 8), min_size=k, max_size=k)), reverse=True)
        S[r, :lens[r]] = np.array(v) / 8.0
    budget = draw(st.integers(0, bs * ld + 2))
    return lens, S, budget


@CASES
@given(case=chains())
def test_allocation_is_the_best_prefix_closed_set(case):
    """[HS] Section 4.4: the budget goes to the highest survivals, each request
    keeps a prefix of its chain, every slot is used while any is left, and the
    row bases count each request's slots plus its bonus row."""
    lens, S, budget = case
    alloc, row_base, total, fl = O.allocate(lens, S, budget)
    assert np.all(alloc >= 0) and np.all(alloc <= lens)
    b = min(budget, int(lens.sum()))
    assert alloc.sum() == b
    vals = np.sort(np.concatenate([S[r, :lens[r]] for r in range(len(lens))]))[::-1]
    got = sum(S[r, :alloc[r]].sum() for r in range(len(lens)))
    assert got == pytest.approx(vals[:b].sum(), abs=1e-12)
    assert np.array_equal(row_base, np.concatenate([[0], np.cumsum(alloc + 1)[:-1]]))
    assert total == b + len(lens)


@CASES
@given(S=st.lists(st.floats(0, 1, width=32), max_size=40), B=st.integers(1, 50),
       c0=st.floats(0.5, 50), p=st.floats(0.01, 2))
def test_size_budget_maximizes_goodput_and_the_library_agrees(S, B, c0, p):
    """[HS] Section 4.3 Eq. (2): b* maximizes G(b) = (B + sum of the b best
    survivals) / (c0 + p b), lambda = G(b*) p; the library's host sizing gives
    the same numbers bit for bit."""
    import draft_verification_spec_amd as L
    s = np.array(S, np.float32)
    b, lam, G = O.size_budget(s, B, c0, p)
    top = np.concatenate([[0.0], np.cumsum(np.sort(s.astype(np.float64))[::-1])])
    g = (B + top) / (c0 + p * np.arange(len(top)))
    assert G[b] == pytest.approx(g.max(), rel=1e-12)
    assert lam == pytest.approx(G[b] * p, rel=1e-15)
    lb, llam, lg = L.spec_size_budget(s, B, c0, p)
    assert (lb, llam, lg) == (b, lam, G[b])


@st.composite
def forests(draw):
    n = draw(st.integers(1, 9))
    parent = [-1] + [draw(st.integers(0, j - 1)) for j in range(1, n)]
    q = [0.0] + [draw(st.sampled_from([0.0, 0.125, 0.25, 0.5, 0.75, 1.0])) for _ in range(1, n)]
    rows = draw(st.integers(1, n + 1))
    return np.array(parent, np.int32), np.array(q, np.float32), rows


@CASES
@given(case=forests())
def test_given_forest_rows_are_a_best_preorder_subtree(case):
    """[AS] Section 3.1, Proposition 1: the rows are parent-closed, hold the
    largest sum of Q of their size, and follow the pre-order of the forest
    with children in index order."""
    parent, q, rows_cap = case
    n = len(parent)
    tok = np.arange(n, dtype=np.int32) + 100
    t = O.tree_forest(tok, parent, q, n, rows_cap)
    k = t["n_rows"]
    assert k == min(rows_cap, n) and t["flag"] == 0
    nodes = [0] + [int(v) - 100 for v in t["node_token"][1:k]]
    pr = t["parent_row"][:k]
    for i in range(1, k):
        assert 0 <= pr[i] < i and parent[nodes[i]] == nodes[pr[i]]
    # pre-order: a row's subtree is the rows that follow it up to the first
    # row whose parent lies before it; siblings appear in index order
    for i in range(1, k):
        kids = [c for c in range(i + 1, k) if pr[c] == i]
        assert kids == sorted(kids, key=lambda c: nodes[c])
    fQ = t["f_Q"]
    best = 0.0
    import itertools
    for comb in itertools.combinations(range(1, n), k - 1):
        s = set(comb) | {0}
        if all(parent[j] in s for j in comb):
            best = max(best, sum(fQ[j] for j in comb))
    assert t["Q"][1:k].sum() == pytest.approx(best, abs=1e-12)


@CASES
@given(bs=st.integers(1, 4), ld=st.integers(0, 5), V=st.integers(2, 12), seed=st.integers(0, 2 ** 31))
def test_greedy_verify_emits_the_argmax_path(bs, ld, V, seed):
    """[LS] Section 2.1 at T = 0: the accepted drafts are a prefix whose tokens
    are their rows' argmax; the next token is the argmax of the row after
    them; the commit appends exactly the emitted tokens."""
    rng = np.random.default_rng(seed)
    z = rng.integers(-3, 4, (bs * (ld + 1), V)).astype(np.float32)   # ties are frequent
    arg = z.argmax(axis=1)   # the lowest index among ties
    n_slots = rng.integers(0, ld + 1, bs).astype(np.int32)
    rb = np.arange(bs, dtype=np.int64) * (ld + 1)
    tokens = np.where(rng.random((bs, max(ld, 1))) < 0.6, arg.reshape(bs, ld + 1)[:, :max(ld, 1)],
                      rng.integers(0, V, (bs, max(ld, 1))))[:, :ld].astype(np.int32).reshape(bs, ld)
    o = O.verify_chain(z, rb, tokens, np.zeros((bs, ld), np.uint8), n_slots, np.zeros((bs, ld), np.float32),
                       np.zeros(bs, np.float32), 0.0)
    ctx = rng.integers(0, V, (bs, 30)).astype(np.int32)
    clen = rng.integers(0, 20, bs).astype(np.int32)
    c2, l2 = O.commit(ctx.copy(), clen.copy(), 30, o["out_tokens"], o["out_num"], o["flags"])
    for r in range(bs):
        acc = 0
        while acc < n_slots[r] and tokens[r, acc] == arg[rb[r] + acc]:
            acc += 1
        assert o["out_accepted"][r] == acc and o["out_num"][r] == acc + 1
        assert np.array_equal(o["out_tokens"][r, :acc], tokens[r, :acc])
        assert o["out_tokens"][r, acc] == arg[rb[r] + acc]
        assert np.array_equal(c2[r, :clen[r]], ctx[r, :clen[r]])
        assert l2[r] == clen[r] + acc + 1
        assert np.array_equal(c2[r, clen[r]:l2[r]], o["out_tokens"][r, :acc + 1])
