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
