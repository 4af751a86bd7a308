"""Oracle pins: n-gram scan (brute force by substring search, planted spans)
and budget allocation (exhaustive subset search, invariants)."""
import itertools

import numpy as np
import pytest

from oracle import oracle as O
from workloads import synth


# ---------------------------------------------------------------------------
# n-gram scan: brute force over a different formulation
# ---------------------------------------------------------------------------

def _occ_ends(s, pat, limit_end):
    """End positions j of every occurrence of ``pat`` in ``s`` with j < limit_end."""
    out = []
    i = s.find(pat)
    while i >= 0:
        j = i + len(pat) - 1
        if j < limit_end:
            out.append(j)
        i = s.find(pat, i + 1)
    return out


def brute_ngram(x, n_min, n_max, L, cap):
    """Search by suffix length with str.find: the longest suffix of the text
    that occurs ending before the last position; among its occurrences the
    latest wins.  The runner-up is the latest other occurrence with the
    largest maximal length."""
    T = len(x)
    s = "".join(chr(65 + int(t)) for t in x)

    def maximal_len(j):
        # largest l (<= cap, <= j+1) such that the suffix of length l ends at j
        best = 0
        for l in range(1, min(cap, j + 1) + 1):
            if s[j - l + 1:j + 1] == s[T - l:]:
                best = l
            else:
                break
        return best

    best_l, best_j = 0, -1
    for l in range(min(cap, T - 1), n_min - 1, -1):
        ends = _occ_ends(s, s[T - l:], T - 1)
        if ends:
            best_l, best_j = l, max(ends)
            break
    if best_j < 0:
        return [], 0, (0, 0, 0, -1)
    ru_j = -1
    for l in range(best_l, n_min - 1, -1):
        ends = [j for j in _occ_ends(s, s[T - l:], T - 1) if j != best_j and maximal_len(j) == l]
        if ends:
            ru_j = max(ends)
            break
    n = min(best_l, n_max)
    full = best_l >= n_max
    a = int(ru_j < 0 or x[ru_j + 1] == x[best_j + 1])
    draft = list(x[best_j + 1: min(best_j + 1 + L, T)])
    return draft, len(draft), (n, a, best_l if full else 0, best_j)


@pytest.mark.parametrize("V", [2, 3, 4])
def test_ngram_bruteforce_tiny_alphabets(V):
    rng = np.random.Generator(np.random.Philox(7 + V))
    cases = 0
    for trial in range(300):
        T = int(rng.integers(1, 65))
        x = rng.integers(0, V, T).astype(np.int32)
        n_min = int(rng.integers(1, 6))
        n_max = int(rng.integers(n_min, 16))
        cap = int(rng.choice([4, 8, 256]))
        L = int(rng.integers(1, 16))
        if n_min > cap:
            continue
        d, dl, f = O.ngram_draft(x[None, :], np.array([T], np.int32), n_min, n_max, L, cap)
        bd, bl, bf = brute_ngram(list(x), n_min, n_max, L, cap)
        assert int(dl[0]) == bl, (x, n_min, n_max, cap)
        assert list(d[0, :bl]) == bd
        assert np.all(d[0, bl:] == -1)
        assert tuple(int(v) for v in f[0]) == bf, (list(x), n_min, n_max, cap)
        cases += 1
    assert cases > 200


def test_ngram_planted_span_found():
    rng = np.random.Generator(np.random.Philox(11))
    V, T, span = 32000, 512, 40
    x = synth.uniform_tokens(rng, T, V)
    src = 100
    x[T - span:] = x[src:src + span]
    d, dl, f = O.ngram_draft(x[None, :], np.array([T], np.int32), 3, 15, 15, 256)
    assert f[0, 3] == src + span - 1                 # best match ends at the source's end
    assert f[0, 0] == 15 and f[0, 2] == span         # full match, copy length 40
    assert list(d[0]) == list(x[src + span: src + span + 15])
    # a single size (n_min = n_max = 3): still the longest, m = 40
    d, dl, f = O.ngram_draft(x[None, :], np.array([T], np.int32), 3, 3, 15, 256)
    assert f[0, 0] == 3 and f[0, 2] == span and f[0, 3] == src + span - 1


def test_ngram_copy_heavy_context_drafts_source():
    c = synth.config1(BS=2, V=1000)
    for r in range(2):
        x, T = c["ctx"][r], int(c["ctx_len"][r])
        d, dl, f = O.ngram_draft(x[None, :], np.array([T], np.int32), 4, 4, 15, 256)
        if dl[0] == 0:
            continue
        j = int(f[0, 3])
        assert np.array_equal(x[j - 3:j + 1], x[T - 4:T])     # the match is real
        assert list(d[0, :dl[0]]) == list(x[j + 1:j + 1 + dl[0]])


def test_ngram_edge_cases():
    # empty / too-short contexts and no match
    x = np.array([[1, 2, 3, 4]], np.int32)
    assert O.ngram_draft(x, np.array([0], np.int32), 1, 3)[1][0] == 0
    assert O.ngram_draft(x, np.array([1], np.int32), 1, 3)[1][0] == 0
    assert O.ngram_draft(x, np.array([4], np.int32), 1, 3)[1][0] == 0
    # all one token: the longest match is the previous position, capped
    x = np.full((1, 600), 7, np.int32)
    d, dl, f = O.ngram_draft(x, np.array([600], np.int32), 5, 15, 15, 256)
    assert f[0, 0] == 15 and f[0, 2] == 256 and f[0, 3] == 598 and dl[0] == 1
    # query text = context ++ extra
    ctx = np.array([[9, 1, 2, 3, 8, 0, 0]], np.int32)
    d, dl, f = O.ngram_draft(ctx, np.array([5], np.int32), 2, 15, 15, 256, query_req=np.array([0], np.int32),
                             extra=np.array([[1, 2]], np.int32), extra_len=np.array([2], np.int32))
    assert f[0, 3] == 2 and list(d[0, :dl[0]]) == [3, 8, 1, 2]


# ---------------------------------------------------------------------------
# n-gram fill's follower fallback (AdaSpark Section 3.3, "N-gram candidates":
# continue the copied passage; when there is none, take the token that most
# often followed the last three tokens)
# ---------------------------------------------------------------------------

def test_follower_fallback_hand_examples():
    # the copy [7, 1, 2, 3] reaches the end of the text; then the last three
    # tokens 1 2 3 were followed by 9 twice and by 7 once -> 9 (count 2), and
    # 2 3 9 was followed by 1 twice -> 1 (count 2)
    x = np.array([[1, 2, 3, 9, 1, 2, 3, 9, 1, 2, 3, 7, 1, 2, 3]], np.int32)
    d, dl, f, fol = O.ngram_draft(x, np.array([15], np.int32), 3, 15, 6, 256, follow_ctx=3)
    assert dl[0] == 6 and list(d[0]) == [7, 1, 2, 3, 9, 1] and list(fol[0]) == [0, 0, 0, 0, 2, 2]
    assert tuple(f[0]) == (3, 0, 0, 10)                    # the copy's own features are unchanged
    d0, dl0, f0 = O.ngram_draft(x, np.array([15], np.int32), 3, 15, 6, 256)   # fallback off
    assert dl0[0] == 4 and list(d0[0, :4]) == [7, 1, 2, 3]
    # no copy (n_min 4): 5 6 7 was followed by 1 and by 2 once each -> the
    # latest, 2; then 6 7 2 -> 5, 7 2 5 -> 6, 2 5 6 -> 7, and round again
    x = np.array([[5, 6, 7, 1, 5, 6, 7, 2, 5, 6, 7]], np.int32)
    d, dl, f, fol = O.ngram_draft(x, np.array([11], np.int32), 4, 15, 6, 256, follow_ctx=3)
    assert list(d[0]) == [2, 5, 6, 7, 2, 5] and list(fol[0]) == [1] * 6 and tuple(f[0]) == (0, 0, 0, -1)
    # a context never seen before has no follower
    x = np.array([[1, 2, 3, 4, 5]], np.int32)
    d, dl, f, fol = O.ngram_draft(x, np.array([5], np.int32), 3, 15, 6, 256, follow_ctx=3)
    assert dl[0] == 0 and np.all(d[0] == -1) and np.all(fol[0] == 0)
    # texts shorter than the context
    assert O.ngram_draft(x, np.array([2], np.int32), 3, 15, 6, 256, follow_ctx=3)[1][0] == 0


def test_follower_fallback_distinct_follower_limit():
    """A context with 1,024 distinct followers still proposes (all seen once:
    the latest wins); with 1,025 the chain ends."""
    for k, want in ((1024, 1), (1025, 0)):
        x = np.concatenate([np.array([0, 0, 0, 5000 + i], np.int32) for i in range(k)] + [np.zeros(3, np.int32)])
        d, dl, f, fol = O.ngram_draft(x[None, :], np.array([len(x)], np.int32), 5, 15, 1, 256, follow_ctx=3)
        assert dl[0] == want
        if want:
            assert d[0, 0] == 5000 + k - 1 and fol[0, 0] == 1


def brute_follow(x, L, F, primary):
    """The fallback written with Counter over str.find occurrences."""
    from collections import Counter
    T = len(x)
    s = "".join(chr(65 + int(t)) for t in x)
    chain = list(primary)
    fol = [0] * len(chain)
    while len(chain) < L and T + len(chain) >= F:
        ctx = (list(x) + chain)[-F:]
        pat = "".join(chr(65 + int(t)) for t in ctx)
        ends = _occ_ends(s, pat, T - 1)
        if not ends:
            break
        cnt = Counter(int(x[j + 1]) for j in ends)
        if len(cnt) > 1024:
            break
        last = {int(x[j + 1]): j for j in ends}
        tok = max(cnt, key=lambda t: (cnt[t], last[t]))
        chain.append(tok)
        fol.append(cnt[tok])
    return chain, fol


@pytest.mark.parametrize("V", [2, 3, 5])
def test_follower_fallback_bruteforce_tiny_alphabets(V):
    rng = np.random.Generator(np.random.Philox(40 + V))
    used = 0
    for trial in range(300):
        T = int(rng.integers(1, 50))
        x = rng.integers(0, V, T).astype(np.int32)
        n_min = int(rng.integers(1, 7))
        L = int(rng.integers(1, 16))
        F = int(rng.integers(1, 5))
        d, dl, f, fol = O.ngram_draft(x[None, :], np.array([T], np.int32), n_min, 15, L, 256, follow_ctx=F)
        bd, _, _ = brute_ngram(list(x), n_min, 15, L, 256)
        chain, bfol = brute_follow(x, L, F, bd)
        assert int(dl[0]) == len(chain), (list(x), n_min, L, F)
        assert list(d[0, :dl[0]]) == chain and list(fol[0, :dl[0]]) == bfol
        assert np.all(d[0, dl[0]:] == -1) and np.all(fol[0, dl[0]:] == 0)
        used += len(chain) > len(bd)
    assert used > 50


# ---------------------------------------------------------------------------
# allocation
# ---------------------------------------------------------------------------

def random_chains(rng, bs, ld, ties=False):
    lens = rng.integers(0, ld + 1, bs).astype(np.int32)
    S = np.zeros((bs, ld))
    for r in range(bs):
        if ties:
            h = rng.choice([0.5, 0.8, 1.0], ld)
        else:
            h = rng.uniform(0.3, 1.0, ld)
        S[r, :lens[r]] = np.cumprod(h)[:lens[r]]
    return lens, S


def test_allocation_is_best_subset_bruteforce():
    rng = np.random.Generator(np.random.Philox(3))
    for trial in range(200):
        bs, ld = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        lens, S = random_chains(rng, bs, ld, ties=trial % 2 == 0)
        slots = [(r, k) for r in range(bs) for k in range(lens[r])]
        b = int(rng.integers(0, len(slots) + 2))
        alloc, rb, total, fl = O.allocate(lens, S, b)
        take = min(b, len(slots))
        assert alloc.sum() == take
        # the chosen set has the largest total survival of any set of that size
        best = max((sum(S[r, k] for r, k in comb) for comb in itertools.combinations(slots, take)), default=0.0)
        chosen = sum(S[r, k] for r in range(bs) for k in range(alloc[r]))
        assert chosen == pytest.approx(best, rel=1e-12, abs=1e-15)
        # every request keeps a prefix; rows = slots + 1
        assert np.all(alloc <= lens)
        assert list(rb) == list(np.concatenate([[0], np.cumsum(alloc + 1)[:-1]]))
        assert total == take + bs


def test_allocation_tie_order():
    # equal survivals: lower position first, then lower request
    S = np.array([[0.5, 0.5, 0.0], [0.5, 0.5, 0.5]])
    lens = np.array([2, 3], np.int32)
    assert list(O.allocate(lens, S, 1)[0]) == [1, 0]
    assert list(O.allocate(lens, S, 2)[0]) == [1, 1]
    assert list(O.allocate(lens, S, 3)[0]) == [2, 1]
    assert list(O.allocate(lens, S, 4)[0]) == [2, 2]
    assert list(O.allocate(lens, S, 0)[0]) == [0, 0]
    assert list(O.allocate(lens, S, 99)[0]) == [2, 3]


def test_allocation_near_flag():
    lens = np.array([1, 1, 1], np.int32)
    # distinct in fp32: the larger wins, both requests at the cut are flagged
    S = np.array([[0.6, 0.0], [0.6 * (1 + 5e-7), 0.0], [0.1, 0.0]])
    alloc, _, _, fl = O.allocate(lens, S, 1)
    assert list(alloc) == [0, 1, 0]
    assert fl[0] & O.ALLOC_NEAR and fl[1] & O.ALLOC_NEAR and not fl[2] & O.ALLOC_NEAR
    # equal once rounded to fp32 (the ranking precision): the tie order decides; still flagged
    S[1, 0] = 0.6 * (1 + 1e-8)
    alloc, _, _, fl = O.allocate(lens, S, 1)
    assert list(alloc) == [1, 0, 0] and fl[0] & O.ALLOC_NEAR and fl[1] & O.ALLOC_NEAR
    # an exact tie is decided by the tie order and not flagged
    S[1, 0] = 0.6
    alloc, _, _, fl = O.allocate(lens, S, 1)
    assert list(alloc) == [1, 0, 0] and not np.any(fl & O.ALLOC_NEAR)
