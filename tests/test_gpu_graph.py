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
