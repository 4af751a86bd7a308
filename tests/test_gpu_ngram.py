"""GPU parity: spec_ngram_draft against the oracle, bit-exact."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import dev, host
from workloads import synth

pytestmark = pytest.mark.gpu


def run_both(ctx, ctx_len, n_min, n_max, L=15, cap=256, query_req=None, extra=None, extra_len=None):
    import torch
    import draft_verification_spec_amd as S
    print(f"ngram: ctx {ctx.shape} n {n_min}..{n_max} L {L} cap {cap} "
          f"queries {None if query_req is None else len(query_req)}", flush=True)
    g = S.spec_ngram_draft(dev(ctx), dev(ctx_len), n_min, n_max, L, cap,
                           query_req=None if query_req is None else dev(query_req),
                           extra=None if extra is None else dev(extra),
                           extra_len=None if extra_len is None else dev(extra_len))
    torch.cuda.synchronize()
    o = O.ngram_draft(ctx, ctx_len, n_min, n_max, L, cap, query_req=query_req, extra=extra, extra_len=extra_len)
    for name, a, b in zip(("draft", "draft_len", "feat"), g, o):
        assert np.array_equal(host(a), b), (name, np.argwhere(host(a) != b)[:5])
    return o


def test_config0_planted_spans():
    c = synth.config0()
    d, dl, f = run_both(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"])
    assert np.all(f[0::2, 2] >= 40)      # live planted span on even requests


@pytest.mark.parametrize("n", [2, 3, 4])
def test_config1_copy_heavy(n):
    c = synth.config1()
    run_both(c["ctx"], c["ctx_len"], n, n)


def test_config2_batch():
    c = synth.config2()
    d, dl, f = run_both(c["ctx"], c["ctx_len"], 5, 15)
    assert (dl[0::2] > 0).mean() > 0.5   # copy-heavy requests mostly match


def test_config3_tree_queries():
    c = synth.config3_inputs()
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    run_both(c["ctx"], c["ctx_len"], 3, 15, query_req=qr, extra=ex, extra_len=el)


def test_config4_zipf_32k():
    c = synth.config4()
    run_both(c["ctx"], c["ctx_len"], 5, 15)


def test_random_tiny_alphabets_and_edges():
    rng = np.random.Generator(np.random.Philox(77))
    for V in (2, 3, 4):
        BS, Tmax = 96, 300
        ctx = rng.integers(0, V, (BS, Tmax)).astype(np.int32)
        ctx_len = rng.integers(0, Tmax + 1, BS).astype(np.int32)
        ctx_len[:4] = [0, 1, 2, Tmax]
        for n_min, n_max, cap, L in ((1, 15, 256, 15), (3, 3, 8, 7), (5, 12, 16, 32), (2, 40, 1024, 1)):
            run_both(ctx, ctx_len, n_min, n_max, L, cap)
    # a context made of one token: capped matches everywhere
    ctx = np.full((3, 5000), 9, np.int32)
    run_both(ctx, np.array([5000, 2049, 2048], np.int32), 5, 15)
    # lengths outside [0, stride] are clamped; out-of-range requests give empty texts
    ctx = rng.integers(0, 3, (4, 64)).astype(np.int32)
    import torch
    import draft_verification_spec_amd as S
    d, dl, f = S.spec_ngram_draft(dev(ctx), dev(np.array([-5, 999, 64, 10], np.int32)), 2, 8, 15, 256,
                                  query_req=dev(np.array([0, 1, 7, -1], np.int32)))
    torch.cuda.synchronize()
    o = O.ngram_draft(ctx, np.array([0, 64, 64, 10], np.int32), 2, 8, 15, 256, query_req=np.array([0, 1, 2, 3], np.int32))
    assert np.array_equal(host(dl)[:2], o[1][:2])
    assert host(dl)[0] == 0 and np.all(host(dl)[2:] == 0) and np.all(host(f)[2:, 3] == -1)


def test_extra_text_long():
    rng = np.random.Generator(np.random.Philox(78))
    ctx = rng.integers(0, 4, (5, 3000)).astype(np.int32)
    ctx_len = np.array([3000, 2500, 10, 0, 2999], np.int32)
    qr = np.array([0, 1, 2, 3, 4, 0, 1], np.int32)
    ex = rng.integers(0, 4, (7, 40)).astype(np.int32)
    el = np.array([40, 0, 17, 40, 1, 3, 39], np.int32)
    run_both(ctx, ctx_len, 2, 15, 15, 256, query_req=qr, extra=ex, extra_len=el)


# ---------------------------------------------------------------------------
# the n-gram fill's follower fallback (follow_ctx > 0)
# ---------------------------------------------------------------------------

def run_follow(ctx, ctx_len, n_min, n_max, L, F, cap=256, query_req=None, extra=None, extra_len=None, tag=""):
    import torch
    import draft_verification_spec_amd as S
    print(f"ngram follow {tag}: ctx {ctx.shape} n {n_min}..{n_max} L {L} F {F} "
          f"queries {None if query_req is None else len(query_req)}", flush=True)
    g = S.spec_ngram_draft(dev(ctx), dev(ctx_len), n_min, n_max, L, cap,
                           query_req=None if query_req is None else dev(query_req),
                           extra=None if extra is None else dev(extra),
                           extra_len=None if extra_len is None else dev(extra_len), follow_ctx=F)
    torch.cuda.synchronize()
    o = O.ngram_draft(ctx, ctx_len, n_min, n_max, L, cap, query_req=query_req, extra=extra, extra_len=extra_len,
                      follow_ctx=F)
    for name, a, b in zip(("draft", "draft_len", "feat", "follow"), g, o):
        assert np.array_equal(host(a), b), (tag, name, np.argwhere(host(a) != b)[:5])
    return o


def test_follow_random_tiny_alphabets():
    """Small alphabets and short texts, where copies often reach the end of
    the text and most contexts have several followers."""
    rng = np.random.Generator(np.random.Philox(91))
    extended = 0
    for V in (2, 3, 5):
        BS, Tmax = 128, 200
        ctx = rng.integers(0, V, (BS, Tmax)).astype(np.int32)
        ctx_len = rng.integers(0, Tmax + 1, BS).astype(np.int32)
        for F, n_min, L in ((3, 3, 15), (1, 4, 32), (4, 2, 7), (8, 5, 20)):
            d, dl, f, fol = run_follow(ctx, ctx_len, n_min, 15, L, F, tag=f"V {V}")
            extended += int((fol > 0).any(axis=1).sum())
    assert extended > 300


def test_follow_window_sizes_and_long_texts():
    """Texts that take each scan window (up to 8,192, 16,384 and 32,768
    tokens) and one longer than the largest (read from memory): periodic
    texts ending in a span written twice, so the copy reaches the end."""
    rng = np.random.Generator(np.random.Philox(92))
    for T in (3000, 12000, 30000, 40000):
        BS = 6
        ctx = np.zeros((BS, T), np.int32)
        for r in range(BS):
            period = int(rng.integers(3, 40))
            base = rng.integers(0, 50, period)
            x = np.resize(base, T).astype(np.int32)
            noise = rng.random(T) < 0.05
            x[noise] = rng.integers(0, 50, int(noise.sum()))
            # the text ends with a fresh span twice: the copy stops at the end
            span = rng.integers(50, 60, int(rng.integers(3, 9))).astype(np.int32)
            x[T - 2 * len(span):] = np.concatenate([span, span])
            ctx[r] = x
        ctx_len = np.full(BS, T, np.int32)
        ctx_len[-1] = T - 7
        d, dl, f, fol = run_follow(ctx, ctx_len, 3, 15, 15, 3, tag=f"T {T}")
        assert (fol[:-1] > 0).any(axis=1).all()


def test_follow_distinct_limit_and_edges():
    rows = []
    for k in (1024, 1025, 3):
        rows.append(np.concatenate([np.array([0, 0, 0, 5000 + i], np.int32) for i in range(k)] +
                                   [np.zeros(3, np.int32)]))
    rows.append(np.array([1, 2, 3, 9, 1, 2, 3, 9, 1, 2, 3, 7, 1, 2, 3], np.int32))
    rows.append(np.array([5, 6, 7, 1, 5, 6, 7, 2, 5, 6, 7], np.int32))
    rows.append(np.array([1, 2], np.int32))
    rows.append(np.zeros(0, np.int32))
    T = max(len(x) for x in rows)
    ctx = np.zeros((len(rows), T), np.int32)
    for i, x in enumerate(rows):
        ctx[i, :len(x)] = x
    ctx_len = np.array([len(x) for x in rows], np.int32)
    d, dl, f, fol = run_follow(ctx, ctx_len, 5, 15, 6, 3, tag="limits")
    assert dl[0] >= 1 and dl[1] == 0
    d, dl, f, fol = run_follow(ctx, ctx_len, 3, 15, 32, 3, tag="limits n_min 3")


def test_follow_tree_queries():
    """The tree workload's n-gram fill (anchor and picks) with the pages'
    three-token follower context."""
    c = synth.config3_inputs()
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    run_follow(c["ctx"], c["ctx_len"], 3, 15, c["L"], 3, query_req=qr, extra=ex, extra_len=el, tag="tree")
