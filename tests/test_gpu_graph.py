"""A HIP-graph capture of the whole step replays to the eager result, replay
after replay, with eager work and synchronisations in between."""
import numpy as np
import pytest

from tests.gpu_helpers import dev
from workloads import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import draft_verification_spec_amd as S
    c = synth.config2(BS=32, V=50000, ctx_extra=32)
    V, BS, L = c["V"], c["BS"], 15
    ctx, ctx_len0 = dev(c["ctx"]), dev(c["ctx_len"])
    ctx_len = ctx_len0.clone()
    target = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, V)
    rb = dev(np.arange(BS, dtype=np.int64) * 16)
    args = dict(model_tokens=dev(c["model_tokens"]), model_conf=dev(c["model_conf_logit"]),
                model_point_mass=dev(c["model_point_mass"]))
    u_acc, u_smp = dev(c["u_acc"][:, :L]), dev(c["u_smp"])
    ws = [torch.empty(1 << 22, dtype=torch.uint8, device="cuda:0") for _ in range(3)]
    bufs = {}

    def step():
        ctx_len.copy_(ctx_len0)
        d, dl, f = S.spec_ngram_draft(ctx, ctx_len, 5, 15, L, 256, out=bufs.get("ng"), workspace=ws[0])
        al = S.spec_allocate_budget(mode="chain", ngram_draft=d, ngram_len=dl, ngram_feat=f, est=c["estimator"],
                                    lam=c["lam"], budget=64, policy="proposed", ld=L, out=bufs.get("al"),
                                    workspace=ws[1], **args)
        out = S.spec_verify_chain(target, rb, al["chain_tokens"], al["alloc_len"], 1.0, u_accept=u_acc,
                                  u_sample=u_smp, slot_flags=al["slot_flags"], out_flags=al["out_flags"], ctx=ctx,
                                  ctx_len=ctx_len, out=bufs.get("vf"), workspace=ws[2])
        bufs.setdefault("ng", (d, dl, f))
        bufs.setdefault("al", al)
        bufs.setdefault("vf", {k: v for k, v in out.items() if k != "out_flags"})
        return out

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
        out = step()
    torch.cuda.synchronize()
    ref = {k: v.cpu().clone() for k, v in out.items()}
    ref_ctx = ctx.cpu().clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for v in out.values():
            v.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v.cpu(), ref[k]), (rep, k)
        assert torch.equal(ctx.cpu(), ref_ctx)
        with torch.cuda.stream(s):
            step()          # eager work between replays
        torch.cuda.synchronize()


def test_tree_step_graph_replays_match_eager():
    """The tree step (n-gram fill with the follower fallback, Eq. (6) tree
    build with S(n), greedy verification with commit) captured in one graph
    replays to the eager result."""
    import torch
    import draft_verification_spec_amd as S
    c = synth.config3_inputs(BS=16, V=50000)
    BS, V, P, Kc, R = c["BS"], c["V"], c["P"], c["Kc"], c["rows_cap"]
    ctx_h = np.zeros((BS, c["ctx"].shape[1] + R), np.int32)
    ctx_h[:, :c["ctx"].shape[1]] = c["ctx"]
    for r in range(BS):                       # texts ending in a repeated span: followers appear
        T = int(c["ctx_len"][r])
        ctx_h[r, T - 8:T] = np.tile(ctx_h[r, T - 12:T - 8], 2)
    ctx, ctx_len = dev(ctx_h), dev(c["ctx_len"])
    ctx_len_new = torch.zeros_like(ctx_len)
    qr, ex, el = synth.tree_queries(ctx_h, c["ctx_len"], c["block"])
    qr, ex, el, block = dev(qr), dev(ex), dev(el), dev(c["block"])
    f = synth.tree_score_inputs(BS, P, Kc)
    sc0 = dict(coef=f["coef"], h=dev(f["h"]), sigma=dev(f["sigma"]), r_share=dev(f["r_share"]),
               psi_ctx=dev(f["psi_ctx"]), b_req=dev(f["b_req"]), p_src=dev(f["p_src"]))
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda:0")
    flags = torch.zeros(BS, dtype=torch.int32, device="cuda:0")
    bufs = {}

    def build():
        d, dl, ft, fol = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], c["L"], 256, query_req=qr,
                                            extra=ex, extra_len=el, out=bufs.get("ng"), follow_ctx=3)
        t = S.spec_allocate_budget(mode="tree", block=block, ngram_draft=d, ngram_len=dl, ngram_follow=fol,
                                   scores=dict(sc0, ngram_feat=ft), c_max=c["c_max"], depth_max=c["depth_max"],
                                   rows_cap=R, s_curve=True, out=bufs.get("tr"))
        bufs.setdefault("ng", (d, dl, ft, fol))
        bufs.setdefault("tr", t)
        return t

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t = build()
    torch.cuda.synchronize()
    assert (bufs["ng"][3] > 0).any()
    rows = synth.tree_target_rows(3, t["node_token"].cpu().numpy(), t["parent_row"].cpu().numpy(),
                                  t["n_rows"].cpu().numpy(), c["truth"], V, R)
    logits = dev(rows).reshape(-1, V)
    rb = dev(np.arange(BS, dtype=np.int64) * R)

    def step():
        tr = build()
        out = S.spec_verify_tree(logits, rb, tr["node_token"], tr["parent_row"], tr["n_rows"], out_flags=flags,
                                 ctx=ctx, ctx_len=ctx_len, ctx_len_out=ctx_len_new, out=bufs.get("vt"),
                                 workspace=ws)
        bufs.setdefault("vt", out)
        return out

    with torch.cuda.stream(s):
        step()
        out = step()
    torch.cuda.synchronize()
    watched = lambda: dict(out, ctx_len_new=ctx_len_new, **{f"ng{i}": v for i, v in enumerate(bufs["ng"])},
                           **{f"tr_{k}": v for k, v in bufs["tr"].items()})
    ref = {k: v.cpu().clone() for k, v in watched().items()}
    ref_ctx = ctx.cpu().clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for k, v in watched().items():
            if k != "out_flags":
                v.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for k, v in watched().items():
            assert torch.equal(v.cpu(), ref[k]), (rep, k)
        assert torch.equal(ctx.cpu(), ref_ctx)
        with torch.cuda.stream(s):
            step()          # eager work between replays
        torch.cuda.synchronize()
