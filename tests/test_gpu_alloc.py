"""GPU parity: spec_allocate_budget (chains and trees) against the oracle, on
the oracle's own upstream n-gram outputs."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import assert_close, assert_rows_equal, dev, host, ok_rows
from workloads import synth

pytestmark = pytest.mark.gpu


def gpu_chain_alloc(model_tokens, conf, conf_is_logit, pm, draft, dlen, feat, est, lam, budget, policy, ld=15):
    import torch
    import draft_verification_spec_amd as S
    print(f"alloc chain: bs {model_tokens.shape[0]} budget {budget} lambda {lam} policy {policy}", flush=True)
    out = S.spec_allocate_budget(mode="chain", model_tokens=dev(model_tokens), model_conf=dev(conf),
                                 ngram_draft=dev(draft), ngram_len=dev(dlen), ngram_feat=dev(feat), est=est,
                                 lam=lam, budget=budget, policy=policy, conf_is_logit=conf_is_logit,
                                 model_point_mass=None if pm is None else dev(pm), ld=ld)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def compare_chain_alloc(g, o, budget):
    ok = ok_rows(o["flags"])
    for k in ("tokens", "slot_flags"):
        assert_rows_equal(g["chain_tokens" if k == "tokens" else k], o[k], ok, k)
    assert_rows_equal(g["chain_len"], o["chain_len"], ok, "chain_len")
    assert_rows_equal(g["chain_src"], o["chain_src"], ok, "chain_src")
    assert_rows_equal(g["alloc_len"], o["alloc_len"], ok, "alloc_len")
    assert_close(g["survival"], o["S"], "survival")
    # row bases: consistent with the GPU's own allocation, equal to the oracle's
    # up to the first excused request
    rb = np.concatenate([[0], np.cumsum(g["alloc_len"] + 1)[:-1]])
    assert np.array_equal(g["row_base"], rb)
    first_bad = np.argmin(ok) if not ok.all() else len(ok)
    assert np.array_equal(g["row_base"][:first_bad + 1][:len(ok)], o["row_base"][:first_bad + 1][:len(ok)])
    assert g["total_rows"][0] == int(g["alloc_len"].sum()) + len(ok)
    if ok.all():
        assert g["total_rows"][0] == o["total_rows"]
    assert g["alloc_len"].sum() == min(budget, int(g["chain_len"].sum()))
    assert np.all(g["alloc_len"] <= g["chain_len"])


@pytest.mark.parametrize("cfg", [2, 4])
def test_chain_alloc_configs(cfg):
    c = synth.config2() if cfg == 2 else synth.config4()
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], 15, 256)
    o = O.allocate_budget(c["model_tokens"], c["model_conf_logit"], True, c["model_point_mass"], draft, dlen, feat,
                          c["estimator"], c["lam"], c["budget"], "proposed", ld=15)
    g = gpu_chain_alloc(c["model_tokens"], c["model_conf_logit"], True, c["model_point_mass"], draft, dlen, feat,
                        c["estimator"], c["lam"], c["budget"], "proposed")
    compare_chain_alloc(g, o, c["budget"])
    print("sources:", np.bincount(g["chain_src"], minlength=4), "flags excused:", (~ok_rows(o["flags"])).sum())


@pytest.mark.parametrize("policy", list(O.POLICIES))
def test_chain_alloc_random_policies(policy):
    rng = np.random.Generator(np.random.Philox(500 + O.POLICIES[policy]))
    bs, K, ld = 300, 7, 15
    truth = rng.integers(0, 50, (bs, 20)).astype(np.int32)
    d = truth[:, :K].copy()
    flip = rng.random((bs, K)) < 0.3
    d[flip] = rng.integers(0, 50, int(flip.sum()))
    dlen = rng.integers(0, 16, bs).astype(np.int32)
    draft = np.full((bs, 15), -1, np.int32)
    for r in range(bs):
        draft[r, :dlen[r]] = truth[r, :dlen[r]] if rng.random() < 0.5 else rng.integers(0, 50, dlen[r])
    draft[:20, :K] = d[:20]                       # contains-rule cases
    dlen[:20] = np.maximum(dlen[:20], K + 1)
    for r in range(20):
        draft[r, K:dlen[r]] = rng.integers(0, 50, dlen[r] - K)
    n = np.where(dlen > 0, rng.integers(5, 16, bs), 0)
    feat = np.stack([n, rng.integers(0, 2, bs), np.where(n >= 15, rng.integers(15, 400, bs), 0),
                     np.full(bs, 3)], 1).astype(np.int32)
    conf = rng.standard_normal((bs, K)).astype(np.float32) + 1
    pm = (rng.random(bs) < 0.5).astype(np.uint8)
    est = synth.estimator_qwen3_4b()
    for budget in (0, 1, 257, 10_000):
        for lam in (0.0, 0.309):
            o = O.allocate_budget(d, conf, True, pm, draft, dlen, feat, est, lam, budget, policy, ld=ld)
            g = gpu_chain_alloc(d, conf, True, pm, draft, dlen, feat, est, lam, budget, policy)
            compare_chain_alloc(g, o, budget)
    # probabilities instead of logits
    probs = (1 / (1 + np.exp(-conf.astype(np.float64)))).astype(np.float32)
    o = O.allocate_budget(d, probs, False, pm, draft, dlen, feat, est, 0.309, 100, policy, ld=ld)
    g = gpu_chain_alloc(d, probs, False, pm, draft, dlen, feat, est, 0.309, 100, policy)
    compare_chain_alloc(g, o, 100)


@pytest.mark.parametrize("bs,ld,gw", [(300, 32, 32), (257, 20, 15), (1, 32, 32), (600, 15, 15), (33, 16, 16)])
def test_chain_alloc_widths_and_key_storage(bs, ld, gw):
    """Chains longer than 16 slots (ld up to 32, n-gram drafts as wide), a
    batch that ends inside a workgroup of the slot pass, one request, and
    batches with more ranking keys than the selection keeps in LDS (bs * ld >
    4096: it reads them from global memory)."""
    rng = np.random.Generator(np.random.Philox(900 + bs + ld))
    K = 7
    truth = rng.integers(0, 40, (bs, gw + 2)).astype(np.int32)
    d = truth[:, :K].copy()
    flip = rng.random((bs, K)) < 0.3
    d[flip] = rng.integers(0, 40, int(flip.sum()))
    dlen = rng.integers(0, gw + 1, bs).astype(np.int32)
    draft = np.full((bs, gw), -1, np.int32)
    for r in range(bs):
        draft[r, :dlen[r]] = truth[r, :dlen[r]] if rng.random() < 0.6 else rng.integers(0, 40, dlen[r])
    n = np.where(dlen > 0, rng.integers(5, 16, bs), 0)
    feat = np.stack([n, rng.integers(0, 2, bs), np.where(n >= 15, rng.integers(15, 400, bs), 0),
                     np.full(bs, 3)], 1).astype(np.int32)
    conf = rng.standard_normal((bs, K)).astype(np.float32) + 1.5
    pm = (rng.random(bs) < 0.5).astype(np.uint8)
    est = synth.estimator_qwen3_4b()
    for budget in (0, 5, bs * 3, 10 ** 6):
        o = O.allocate_budget(d, conf, True, pm, draft, dlen, feat, est, 0.2, budget, "proposed", ld=ld)
        g = gpu_chain_alloc(d, conf, True, pm, draft, dlen, feat, est, 0.2, budget, "proposed", ld=ld)
        compare_chain_alloc(g, o, budget)


def test_tree_build_config3():
    import torch
    import draft_verification_spec_amd as S
    c = synth.config3_inputs()
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], c["L"], 256,
                                      query_req=qr, extra=ex, extra_len=el)
    o = O.tree_build_batch(c["block"], draft, dlen, c["w_node"], c["w_none"], c["depth_max"], c["rows_cap"])
    print("tree build: bs", c["BS"], "forest sizes", o["count"].min(), o["count"].max(), flush=True)
    g = S.spec_allocate_budget(mode="tree", block=dev(c["block"]), ngram_draft=dev(draft), ngram_len=dev(dlen),
                               w_node=dev(c["w_node"]), w_none=dev(c["w_none"]), depth_max=c["depth_max"],
                               rows_cap=c["rows_cap"])
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    ok = ok_rows(o["flags"])
    assert_rows_equal(g["forest_count"], o["count"], np.ones(len(ok), bool), "forest_count")
    for k in ("node_token", "parent_row", "n_rows"):
        assert_rows_equal(g[k], o[k], ok, k)
    assert_close(g["Q"], o["Q"], "Q")
    if ok.all():
        assert np.array_equal(g["row_base"], o["row_base"])
    assert g["total_rows"][0] == g["n_rows"].sum()
    # small random forests, all row caps
    rng = np.random.Generator(np.random.Philox(9))
    BS, P, Kc, L = 40, 3, 3, 6
    block = np.stack([np.stack([rng.choice(8, Kc, replace=False) for _ in range(P)]) for _ in range(BS)]).astype(np.int32)
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    ng = rng.integers(0, 8, (BS * (P + 1), L)).astype(np.int32)
    cm = 1 + P * Kc + (P + 1) * L
    wn = rng.standard_exponential((BS, cm)).astype(np.float32)
    wz = rng.standard_exponential((BS, cm)).astype(np.float32)
    for rows_cap in (1, 2, 5, 16, 40):
        for dmax in (1, 2, 32):
            o = O.tree_build_batch(block, ng, ngl, wn, wz, dmax, rows_cap)
            g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                       w_node=dev(wn), w_none=dev(wz), depth_max=dmax, rows_cap=rows_cap)
            torch.cuda.synchronize()
            g = {k: host(v) for k, v in g.items()}
            ok = ok_rows(o["flags"])
            for k in ("node_token", "parent_row", "n_rows"):
                assert_rows_equal(g[k], o[k], ok, f"{k} cap {rows_cap} depth {dmax}")
            assert_close(g["Q"], o["Q"], "Q")


@pytest.mark.parametrize("c_max", [61, 64, 65, 130, 256, 257, 600, 1024])
def test_tree_build_large_forests(c_max):
    """Forests that fill one, several or all of the forest's 64-node groups,
    chains longer than 64 tokens, and the c_max cap reached mid-chain."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(31 + c_max))
    BS, P, Kc, L, vocab = 24, 15, 4, 70, 40
    block = np.stack([np.stack([rng.choice(vocab, Kc, replace=False) for _ in range(P)])
                      for _ in range(BS)]).astype(np.int32)
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    ng = rng.integers(0, vocab, (BS * (P + 1), L)).astype(np.int32)
    # half the chains repeat an earlier chain's prefix, so they descend first
    for q in range(BS * (P + 1)):
        if q % (P + 1) and rng.random() < 0.5:
            src = q - 1 - int(rng.integers(0, q % (P + 1)))
            k = int(rng.integers(1, L))
            ng[q, :k] = ng[src, :k]
    wn = rng.standard_exponential((BS, c_max)).astype(np.float32)
    wz = rng.standard_exponential((BS, c_max)).astype(np.float32)
    for dmax, rows_cap in ((100, 64), (32, 16)):
        print(f"tree build: c_max {c_max} depth {dmax} rows_cap {rows_cap}", flush=True)
        o = O.tree_build_batch(block, ng, ngl, wn, wz, dmax, rows_cap)
        g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                   w_node=dev(wn), w_none=dev(wz), depth_max=dmax, rows_cap=rows_cap)
        torch.cuda.synchronize()
        g = {k: host(v) for k, v in g.items()}
        ok = ok_rows(o["flags"])
        assert_rows_equal(g["forest_count"], o["count"], np.ones(BS, bool), "forest_count")
        for k in ("node_token", "parent_row", "n_rows"):
            assert_rows_equal(g[k], o[k], ok, f"{k} c_max {c_max} depth {dmax}")
        assert_close(g["Q"], o["Q"], "Q")
    if c_max <= 257:
        assert o["count"].max() == c_max   # the cap is reached


@pytest.mark.parametrize("prior_only", [True, False])
def test_tree_build_eq6_scores_and_s_curve(prior_only):
    """The tree build with the Eq. (6) scores computed on the device from the
    drafter's and the n-gram chains' features (AdaSpark Section 3.3), and the
    S(n) curve of the best-first order (Section 3.1), on the tree workload."""
    import torch
    import draft_verification_spec_amd as S
    c = synth.config3_inputs()
    BS, P, Kc = c["BS"], c["P"], c["Kc"]
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], c["L"], 256,
                                      query_req=qr, extra=ex, extra_len=el)
    f = synth.tree_score_inputs(BS, P, Kc, prior_only=prior_only)
    per = [dict(coef=f["coef"], h=f["h"][r], sigma=f["sigma"][r], r_share=f["r_share"][r],
                psi_ctx=f["psi_ctx"][r], b_req=f["b_req"][r], p_src=f["p_src"][r],
                ng_feat=feat.reshape(BS, P + 1, 4)[r]) for r in range(BS)]
    o = O.tree_build_batch(c["block"], draft, dlen, depth_max=c["depth_max"], rows_cap=c["rows_cap"], scores=per,
                           c_max=c["c_max"])
    sc = dict(coef=f["coef"], h=dev(f["h"]), sigma=dev(f["sigma"]), r_share=dev(f["r_share"]),
              psi_ctx=dev(f["psi_ctx"]), b_req=dev(f["b_req"]), p_src=dev(f["p_src"]), ngram_feat=dev(feat))
    g = S.spec_allocate_budget(mode="tree", block=dev(c["block"]), ngram_draft=dev(draft), ngram_len=dev(dlen),
                               scores=sc, c_max=c["c_max"], depth_max=c["depth_max"], rows_cap=c["rows_cap"],
                               s_curve=True)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    ok = ok_rows(o["flags"])
    assert_rows_equal(g["forest_count"], o["count"], np.ones(len(ok), bool), "forest_count")
    for k in ("node_token", "parent_row", "n_rows"):
        assert_rows_equal(g[k], o[k], ok, k)
    assert_close(g["Q"], o["Q"], "Q")
    assert_close(g["s_curve"], o["S_curve"], "S(n)")
    # the curve at the built width is the tree's own sum of Q
    for r in range(BS):
        n = g["n_rows"][r]
        assert g["s_curve"][r, n - 1] == pytest.approx(g["Q"][r, 1:n].sum(), rel=1e-5)
    print(f"  S(16) mean {g['s_curve'][:, -1].mean():.3f}, excused {np.mean(~ok):.3f}")


def test_tree_build_follower_buckets():
    """Chains whose tokens mix copies and follower-fallback tokens (follower
    counts 1..300, every evidence class), scored with Eq. (6): the follower
    buckets 32..63, their agreements and contradictions, on random forests
    and on the tree workload with its texts ending in a repeated span."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(55))
    BS, P, Kc, L, vocab = 40, 6, 3, 20, 12
    block = np.stack([np.stack([rng.choice(vocab, Kc, replace=False) for _ in range(P)])
                      for _ in range(BS)]).astype(np.int32)
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    ng = rng.integers(0, vocab, (BS * (P + 1), L)).astype(np.int32)
    fol = np.where(rng.random((BS * (P + 1), L)) < 0.5, 0, rng.integers(1, 300, (BS * (P + 1), L))).astype(np.int32)
    feat = np.zeros((BS * (P + 1), 4), np.int32)
    feat[:, 0] = rng.integers(1, 16, BS * (P + 1))
    feat[:, 2] = np.where(rng.random(BS * (P + 1)) < 0.5, rng.integers(15, 300, BS * (P + 1)), 0)
    c_max = 1 + P * Kc + (P + 1) * L
    f = synth.tree_score_inputs(BS, P, Kc)
    cases = [("random", block, ng, ngl, fol, feat, f, c_max, 64, 40)]
    c = synth.config3_inputs()
    ctx = c["ctx"].copy()
    for r in range(c["BS"]):
        T = int(c["ctx_len"][r])
        span = rng.integers(0, c["V"], 6).astype(np.int32)
        ctx[r, T - 12:T] = np.concatenate([span, span])
    qr, ex, el = synth.tree_queries(ctx, c["ctx_len"], c["block"])
    d3, l3, f3, fol3 = O.ngram_draft(ctx, c["ctx_len"], c["n_min"], c["n_max"], c["L"], 256,
                                     query_req=qr, extra=ex, extra_len=el, follow_ctx=3)
    assert (fol3 > 0).any()
    f3s = synth.tree_score_inputs(c["BS"], c["P"], c["Kc"])
    cases.append(("tree workload", c["block"], d3, l3, fol3, f3, f3s, c["c_max"], c["depth_max"], c["rows_cap"]))
    for tag, blk, d, dl, fl, ft, fs, cm, dmax, rows_cap in cases:
        bs, p_, kc = blk.shape
        print(f"tree build with followers ({tag}): bs {bs} c_max {cm}", flush=True)
        per = [dict(coef=fs["coef"], h=fs["h"][r], sigma=fs["sigma"][r], r_share=fs["r_share"][r],
                    psi_ctx=fs["psi_ctx"][r], b_req=fs["b_req"][r], p_src=fs["p_src"][r],
                    ng_feat=ft.reshape(bs, p_ + 1, 4)[r]) for r in range(bs)]
        o = O.tree_build_batch(blk, d, dl, depth_max=dmax, rows_cap=rows_cap, scores=per, c_max=cm, ng_follow=fl)
        sc = dict(coef=fs["coef"], h=dev(fs["h"]), sigma=dev(fs["sigma"]), r_share=dev(fs["r_share"]),
                  psi_ctx=dev(fs["psi_ctx"]), b_req=dev(fs["b_req"]), p_src=dev(fs["p_src"]), ngram_feat=dev(ft))
        g = S.spec_allocate_budget(mode="tree", block=dev(blk), ngram_draft=dev(d), ngram_len=dev(dl),
                                   ngram_follow=dev(fl), scores=sc, c_max=cm, depth_max=dmax, rows_cap=rows_cap,
                                   s_curve=True)
        torch.cuda.synchronize()
        g = {k: host(v) for k, v in g.items()}
        ok = ok_rows(o["flags"])
        assert_rows_equal(g["forest_count"], o["count"], np.ones(bs, bool), "forest_count")
        for k in ("node_token", "parent_row", "n_rows"):
            assert_rows_equal(g[k], o[k], ok, f"{k} ({tag})")
        assert_close(g["Q"], o["Q"], "Q")
        assert_close(g["s_curve"], o["S_curve"], "S(n)")
        # the follower weights matter: without the counts the oracle builds other trees
        o0 = O.tree_build_batch(blk, d, dl, depth_max=dmax, rows_cap=rows_cap, scores=per, c_max=cm)
        assert not np.allclose(o0["Q"], o["Q"])


@pytest.mark.parametrize("P,Kc,L,vocab", [(8, 4, 15, 6), (20, 2, 12, 5), (63, 1, 8, 4), (5, 3, 40, 3)])
def test_tree_build_shared_paths(P, Kc, L, vocab):
    """Chains that follow the drafter's picks and then one another's n-gram
    nodes (AdaSpark Section 3.1: a chain extends the forest where its tokens
    leave the existing paths): each request has a text; the picks mostly
    follow it, the siblings are random (duplicates allowed); chain c is mostly
    the text's continuation from pick c, sometimes with one token changed, else
    random.  Small vocabularies make sibling matches and shared continuations
    common.  c_max caps from a few nodes past the block to unbounded, depth
    limits, given weights and Eq. (6) scores with follower counts."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(4100 + 7 * P + Kc))
    BS = 48
    tr = rng.integers(0, vocab, (BS, P + L + 8)).astype(np.int32)
    block = rng.integers(0, vocab, (BS, P, Kc)).astype(np.int32)
    follow = rng.random((BS, P)) < 0.8
    block[:, :, 0] = np.where(follow, tr[:, :P], block[:, :, 0])
    ng = rng.integers(0, vocab, (BS * (P + 1), L)).astype(np.int32)
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    for r in range(BS):
        for c in range(P + 1):
            q = r * (P + 1) + c
            u = rng.random()
            if u < 0.7:
                ng[q] = tr[r, c:c + L]
                if rng.random() < 0.3:
                    j = int(rng.integers(0, L))
                    ng[q, j] = (ng[q, j] + 1) % vocab
    fol = np.where(rng.random((BS * (P + 1), L)) < 0.6, 0, rng.integers(1, 300, (BS * (P + 1), L))).astype(np.int32)
    feat = np.zeros((BS * (P + 1), 4), np.int32)
    feat[:, 0] = rng.integers(1, 16, BS * (P + 1))
    feat[:, 2] = np.where(rng.random(BS * (P + 1)) < 0.5, rng.integers(15, 300, BS * (P + 1)), 0)
    nd = 1 + P * Kc
    full = nd + (P + 1) * L
    f = synth.tree_score_inputs(BS, P, Kc)
    per = [dict(coef=f["coef"], h=f["h"][r], sigma=f["sigma"][r], r_share=f["r_share"][r], psi_ctx=f["psi_ctx"][r],
                b_req=f["b_req"][r], p_src=f["p_src"][r], ng_feat=feat.reshape(BS, P + 1, 4)[r]) for r in range(BS)]
    sc = dict(coef=f["coef"], h=dev(f["h"]), sigma=dev(f["sigma"]), r_share=dev(f["r_share"]),
              psi_ctx=dev(f["psi_ctx"]), b_req=dev(f["b_req"]), p_src=dev(f["p_src"]), ngram_feat=dev(feat))
    shared = 0
    for c_max in sorted({nd + 3, nd + 10, min(full, 512), max(full, 513)}):
        wn = rng.standard_exponential((BS, c_max)).astype(np.float32)
        wz = rng.standard_exponential((BS, c_max)).astype(np.float32)
        for dmax, rows_cap in ((64, 64), (P // 2 + 3, 16), (3, 8)):
            for scored in (False, True):
                print(f"tree build, shared paths: P {P} Kc {Kc} L {L} c_max {c_max} depth {dmax} rows_cap {rows_cap}"
                      f" scored {scored}", flush=True)
                if scored:
                    o = O.tree_build_batch(block, ng, ngl, depth_max=dmax, rows_cap=rows_cap, scores=per, c_max=c_max,
                                           ng_follow=fol)
                    g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                               ngram_follow=dev(fol), scores=sc, c_max=c_max, depth_max=dmax,
                                               rows_cap=rows_cap, s_curve=True)
                else:
                    o = O.tree_build_batch(block, ng, ngl, wn, wz, dmax, rows_cap)
                    g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                               w_node=dev(wn), w_none=dev(wz), depth_max=dmax, rows_cap=rows_cap)
                torch.cuda.synchronize()
                g = {k: host(v) for k, v in g.items()}
                ok = ok_rows(o["flags"])
                assert_rows_equal(g["forest_count"], o["count"], np.ones(BS, bool), f"forest_count c_max {c_max}")
                for k in ("node_token", "parent_row", "n_rows"):
                    assert_rows_equal(g[k], o[k], ok, f"{k} c_max {c_max} depth {dmax} scored {scored}")
                assert_close(g["Q"], o["Q"], "Q")
                if scored:
                    assert_close(g["s_curve"], o["S_curve"], "S(n)")
                if c_max >= full and dmax == 64:
                    # without caps, a forest smaller than the block plus every
                    # chain token: chains passed nodes that were there already
                    shared += int((o["count"] < nd + ngl.reshape(BS, P + 1).sum(1)).sum())
    assert shared > 0


@pytest.mark.parametrize("P,Kc,L,extra", [(0, 1, 6, 0), (0, 3, 6, 4), (4, 1, 6, 0), (3, 2, 0, 0), (3, 2, 5, 0)])
def test_tree_build_degenerate_shapes(P, Kc, L, extra):
    """Shapes at the edges of the tree build's arguments: no drafter block
    (the anchor's chain alone), one candidate per position, no n-gram tokens
    (ngram_ld 0), every chain empty, c_max leaving no room past the block or
    only `extra` nodes, depth limit 1 and a single row."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(7700 + 100 * P + 10 * Kc + L))
    BS, vocab = 24, 4
    block = rng.integers(0, vocab, (BS, P, Kc)).astype(np.int32)
    ng = rng.integers(0, vocab, (BS * (P + 1), L)).astype(np.int32)
    for r in range(BS):
        for c in range(P + 1):
            if P and c < P and L and rng.random() < 0.5:
                ng[r * (P + 1) + c, 0] = block[r, c, 0]   # follow the next pick
    nd = 1 + P * Kc
    for empty in (False, True):
        ngl = np.zeros(BS * (P + 1), np.int32) if empty or L == 0 else rng.integers(0, L + 1, BS * (P + 1)).astype(
            np.int32)
        for c_max in sorted({nd, nd + extra, nd + (P + 1) * L}):
            wn = rng.standard_exponential((BS, c_max)).astype(np.float32)
            wz = rng.standard_exponential((BS, c_max)).astype(np.float32)
            for dmax, rows_cap in ((1, 1), (1, 8), (6, 64)):
                print(f"tree build, edge shape: P {P} Kc {Kc} L {L} empty {empty} c_max {c_max} depth {dmax} "
                      f"rows_cap {rows_cap}", flush=True)
                o = O.tree_build_batch(block, ng, ngl, wn, wz, dmax, rows_cap)
                g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                           w_node=dev(wn), w_none=dev(wz), depth_max=dmax, rows_cap=rows_cap)
                torch.cuda.synchronize()
                g = {k: host(v) for k, v in g.items()}
                ok = ok_rows(o["flags"])
                assert_rows_equal(g["forest_count"], o["count"], np.ones(BS, bool), "forest_count")
                for k in ("node_token", "parent_row", "n_rows"):
                    assert_rows_equal(g[k], o[k], ok, f"{k} c_max {c_max} depth {dmax} rows_cap {rows_cap}")
                assert_close(g["Q"], o["Q"], "Q")
                assert np.array_equal(g["row_base"], np.concatenate([[0], np.cumsum(g["n_rows"])[:-1]]))


def test_tree_build_random_sweep():
    """400 random tree builds (AdaSpark Sections 3.1 and 3.3) against the
    oracle: 0 to 20 positions, 1 to 4 candidates, chains of up to 40 tokens
    that mostly continue a text from each pick (picks mostly follow it),
    vocabularies of 2 to 6 tokens, c_max from the block's size to 1,024 (both
    chain walks), depth limits, 1 to 64 rows, given weights or Eq. (6)
    scores with follower counts."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.default_rng(20261203)
    BS, done = 16, 0
    while done < 400:
        P, Kc, L, V = int(rng.integers(0, 21)), int(rng.integers(1, 5)), int(rng.integers(0, 41)), int(rng.integers(2, 7))
        if (P + 1) * L > 2048:
            continue
        text = rng.integers(0, V, (BS, P + L + 8))
        block = rng.integers(0, V, (BS, P, Kc)).astype(np.int32)
        if P:
            block[:, :, 0] = np.where(rng.random((BS, P)) < 0.8, text[:, :P], block[:, :, 0])
        ng = rng.integers(0, V, (BS * (P + 1), L)).astype(np.int32)
        for r in range(BS):
            for c in range(P + 1):
                if L and rng.random() < 0.7:
                    ng[r * (P + 1) + c] = text[r, c:c + L]
        ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
        nd = 1 + P * Kc
        c_max = max(nd, int(min(1024, rng.choice([nd + (P + 1) * L, nd + int(rng.integers(0, 30)), 1024]))))
        dmax = int(rng.choice([64, int(rng.integers(1, 12))]))
        rows_cap = int(rng.choice([1, 2, 8, 16, 24, 64]))
        scored = P > 0 and bool(rng.random() < 0.5)
        tag = f"P {P} Kc {Kc} L {L} V {V} c_max {c_max} depth {dmax} rows {rows_cap} scored {scored}"
        if done % 50 == 0:
            print(f"tree build, random sweep {done}: {tag}", flush=True)
        if scored:
            fol = np.where(rng.random((BS * (P + 1), L)) < 0.6, 0, rng.integers(1, 300, (BS * (P + 1), L))).astype(
                np.int32)
            feat = np.zeros((BS * (P + 1), 4), np.int32)
            feat[:, 0] = rng.integers(1, 16, BS * (P + 1))
            f = synth.tree_score_inputs(BS, P, Kc)
            per = [dict(coef=f["coef"], h=f["h"][r], sigma=f["sigma"][r], r_share=f["r_share"][r],
                        psi_ctx=f["psi_ctx"][r], b_req=f["b_req"][r], p_src=f["p_src"][r],
                        ng_feat=feat.reshape(BS, P + 1, 4)[r]) for r in range(BS)]
            sc = dict(coef=f["coef"], h=dev(f["h"]), sigma=dev(f["sigma"]), r_share=dev(f["r_share"]),
                      psi_ctx=dev(f["psi_ctx"]), b_req=dev(f["b_req"]), p_src=dev(f["p_src"]), ngram_feat=dev(feat))
            o = O.tree_build_batch(block, ng, ngl, depth_max=dmax, rows_cap=rows_cap, scores=per, c_max=c_max,
                                   ng_follow=fol)
            g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                       ngram_follow=dev(fol), scores=sc, c_max=c_max, depth_max=dmax,
                                       rows_cap=rows_cap, s_curve=True)
        else:
            wn = rng.standard_exponential((BS, c_max)).astype(np.float32)
            wz = rng.standard_exponential((BS, c_max)).astype(np.float32)
            o = O.tree_build_batch(block, ng, ngl, wn, wz, dmax, rows_cap)
            g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                                       w_node=dev(wn), w_none=dev(wz), depth_max=dmax, rows_cap=rows_cap)
        torch.cuda.synchronize()
        g = {k: host(v) for k, v in g.items()}
        ok = ok_rows(o["flags"])
        assert_rows_equal(g["forest_count"], o["count"], np.ones(BS, bool), f"forest_count ({tag})")
        for k in ("node_token", "parent_row", "n_rows"):
            assert_rows_equal(g[k], o[k], ok, f"{k} ({tag})")
        assert_close(g["Q"], o["Q"], f"Q ({tag})")
        done += 1


@pytest.mark.parametrize("BS", [1, 63, 1000, 1024, 1025, 1500])
def test_tree_row_bases_any_batch(BS):
    """Row bases and the total over every batch size the row scan handles in
    registers (up to 1,024 requests) and beyond."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(70 + BS))
    P, Kc, L = 2, 2, 4
    block = rng.integers(0, 6, (BS, P, Kc)).astype(np.int32)
    block[:, :, 1] = (block[:, :, 0] + 1) % 6
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    ng = rng.integers(0, 6, (BS * (P + 1), L)).astype(np.int32)
    cm = 1 + P * Kc + (P + 1) * L
    wn = rng.standard_exponential((BS, cm)).astype(np.float32)
    wz = rng.standard_exponential((BS, cm)).astype(np.float32)
    print(f"tree row bases: bs {BS}", flush=True)
    o = O.tree_build_batch(block, ng, ngl, wn, wz, 8, 6)
    g = S.spec_allocate_budget(mode="tree", block=dev(block), ngram_draft=dev(ng), ngram_len=dev(ngl),
                               w_node=dev(wn), w_none=dev(wz), depth_max=8, rows_cap=6)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    ok = ok_rows(o["flags"])
    assert_rows_equal(g["n_rows"], o["n_rows"], ok, "n_rows")
    rb = np.concatenate([[0], np.cumsum(g["n_rows"])[:-1]]).astype(np.int64)
    assert np.array_equal(g["row_base"], rb)
    assert g["total_rows"][0] == g["n_rows"].sum()
    if ok.all():
        assert np.array_equal(g["row_base"], o["row_base"])


def random_forests(rng, BS, c_max, tie_q=False, shape="random"):
    """Caller-built forests: parents below their children, q in [0, 1]."""
    token = rng.integers(0, 1000, (BS, c_max)).astype(np.int32)
    parent = np.full((BS, c_max), -1, np.int32)
    n = rng.integers(1, c_max + 1, BS).astype(np.int32)
    n[: min(BS, 3)] = c_max
    j = np.arange(1, c_max)
    if c_max > 1:
        if shape == "chain":
            parent[:, 1:] = j - 1
        elif shape == "star":
            parent[:, 1:] = 0
        else:
            parent[:, 1:] = (rng.random((BS, c_max - 1)) * j).astype(np.int32)
    if tie_q:
        q = rng.choice(np.float32([0.0, 0.25, 0.5, 1.0]), (BS, c_max))
    else:
        q = rng.random((BS, c_max)).astype(np.float32)
    return token, parent, q.astype(np.float32), n


def gpu_tree_forest(token, parent, q, n, rows_cap):
    import torch
    import draft_verification_spec_amd as S
    print(f"tree from a given forest: bs {token.shape[0]} c_max {token.shape[1]} rows_cap {rows_cap}", flush=True)
    g = S.spec_allocate_budget(mode="tree", forest=(dev(token), dev(parent), dev(q), dev(n)), rows_cap=rows_cap,
                               s_curve=True)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def compare_tree_forest(g, o):
    """The same fp64 path products and fp32 keys on both sides: every output
    is compared exactly, near ties included."""
    assert np.array_equal(g["forest_count"], o["count"])
    assert np.array_equal(g["out_flags"].astype(np.uint32), o["flags"] & ~np.uint32(O.NEAR_MASK))
    for k in ("node_token", "parent_row", "n_rows", "row_base"):
        assert_rows_equal(g[k], o[k], np.ones(len(o["n_rows"]), bool), k)
    assert np.array_equal(g["Q"], o["Q"].astype(np.float32))
    assert np.array_equal(g["s_curve"], o["S_curve"].astype(np.float32))
    assert g["total_rows"][0] == o["n_rows"].sum()


@pytest.mark.parametrize("c_max", [1, 2, 63, 64, 65, 200, 1024])
def test_tree_from_given_forest(c_max):
    """Forests a caller built (any drafter's, AdaSpark Section 3.1): random,
    chain and star shapes, tied estimates, every row cap."""
    rng = np.random.Generator(np.random.Philox(4400 + c_max))
    for shape in ("random", "chain", "star"):
        for tie_q in (False, True):
            token, parent, q, n = random_forests(rng, 97, c_max, tie_q, shape)
            for rows_cap in (1, 2, 16, 64):
                o = O.tree_forest_batch(token, parent, q, n, rows_cap)
                g = gpu_tree_forest(token, parent, q, n, rows_cap)
                compare_tree_forest(g, o)


def test_tree_from_given_forest_broken_rules():
    """A parent not below its child, q outside [0, 1] or NaN: the request keeps
    the anchor alone and is flagged; node counts outside [1, c_max] are
    clamped and flagged; the other requests are unaffected."""
    rng = np.random.Generator(np.random.Philox(4500))
    BS, c_max = 64, 150
    token, parent, q, n = random_forests(rng, BS, c_max)
    n[:] = c_max
    parent[1, 7] = 7
    parent[2, 100] = 120
    parent[3, 5] = -1
    q[4, 9] = 1.5
    q[5, 140] = -0.25
    q[6, 77] = np.nan
    q[7, 3] = np.inf
    n[8], n[9], n[10] = 0, -5, c_max + 1
    parent[11, c_max - 1] = c_max   # past the node count of request 11 only
    n[11] = c_max - 1
    o = O.tree_forest_batch(token, parent, q, n, 16)
    assert all(o["flags"][r] == O.BAD_FOREST for r in range(1, 8))
    assert all(o["flags"][r] == O.BAD_LENGTH for r in (8, 9, 10))
    assert o["flags"][11] == 0 and o["flags"][0] == 0
    g = gpu_tree_forest(token, parent, q, n, 16)
    compare_tree_forest(g, o)
