"""The host's budget sizing loop over several steps (Hybrid Spark, Section 2
"Asynchronous scheduling", Section 4.4 and Appendix O).

Every step's survivals are copied to pinned host memory asynchronously; the
host sizes the budget b* and the slot price lambda = G(b*) p of step t from
the survivals of step t - 2 and passes them to the allocation as launch
scalars, so nothing waits on the GPU within a step.  The stand-in target
model and drafter put their planted rows and chains in place on the device
from the committed context lengths, so the loop reads nothing back either.
Checked: the scalars of every step are the oracle's sizing of the survivals
two steps prior (bit-exact), and the whole loop (draft, select, allocate,
verify at T = 0, commit) matches the oracle run step by step with the same
scalars."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import assert_close, assert_rows_equal, dev, host, ok_rows
from workloads import synth

pytestmark = pytest.mark.gpu

P_SLOT = 0.3   # cost model C(b) = BS + 0.3 b, in units of one request's decode


def test_async_sizing_loop_matches_oracle():
    import torch
    import draft_verification_spec_amd as S
    loop = synth.ServingLoop()
    BS, V, K, rows, L, T0 = loop.BS, loop.V, loop.K, loop.rows, 15, loop.T_prompt
    est = synth.estimator_linear_length()
    print(f"sizing loop: bs {BS} V {V} steps {loop.steps}", flush=True)
    raws = [loop.step_raw(t) for t in range(loop.steps)]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        ctx, ctx_len = dev(loop.ctx), dev(loop.ctx_len)
        stream_d = dev(loop.stream).long()
        raw_d = [{k: dev(v) for k, v in r.items()} for r in raws]
        row_base = dev(np.arange(BS, dtype=np.int64) * rows)
        pm = dev(np.ones(BS, np.uint8))
        ar = torch.arange(rows, device="cuda:0")
        ring = [torch.empty((BS, L), dtype=torch.float32).pin_memory() for _ in range(3)]
        ev = [torch.cuda.Event() for _ in range(3)]
        b, lam = BS, 0.309   # the first two steps have no survivals two steps back
        rec = []
        for t in range(loop.steps):
            s_host = None
            if t >= 2:
                ev[(t - 2) % 3].synchronize()   # the copy of step t - 2, enqueued two steps ago
                s_host = ring[(t - 2) % 3].numpy().copy()
                b, lam, _ = S.spec_size_budget(s_host, BS, float(BS), P_SLOT)
            # the stand-ins' inputs, put in place on the device
            emitted = (ctx_len - T0).long()
            truth = torch.gather(stream_d, 1, emitted[:, None] + ar[None, :])
            model = torch.where(raw_d[t]["agree"], truth[:, :K], raw_d[t]["rand"].long()).int().contiguous()
            target = raw_d[t]["noise"].clone()
            target.scatter_(2, truth[:, :, None], synth.PLANT_LOGIT)
            target = target.reshape(BS * rows, V)
            d, dl, f = S.spec_ngram_draft(ctx, ctx_len, 5, 15, L, 256)
            al = S.spec_allocate_budget(mode="chain", model_tokens=model, model_conf=raw_d[t]["conf"],
                                        ngram_draft=d, ngram_len=dl, ngram_feat=f, est=est, lam=lam, budget=b,
                                        policy="proposed", conf_is_logit=True, model_point_mass=pm, ld=L)
            ring[t % 3].copy_(al["survival"], non_blocking=True)
            ev[t % 3].record(st)
            snap = {k: v.clone() for k, v in al.items()}
            out = S.spec_verify_chain(target, row_base, al["chain_tokens"], al["alloc_len"], 0.0,
                                      slot_flags=al["slot_flags"], out_flags=al["out_flags"], ctx=ctx,
                                      ctx_len=ctx_len)
            rec.append(dict(b=b, lam=lam, s_host=s_host, al=snap,
                            out={k: v.clone() for k, v in out.items()}, ctx_len=ctx_len.clone()))
        torch.cuda.synchronize()
    rec = [dict(r, al={k: host(v) for k, v in r["al"].items()}, out={k: host(v) for k, v in r["out"].items()},
                ctx_len=host(r["ctx_len"])) for r in rec]
    ctx_g = host(ctx)

    # the scalars: the oracle's sizing of the survivals two steps prior, from
    # the very bytes the allocation wrote
    sizes = []
    for t in range(2, loop.steps):
        s_prev = rec[t - 2]["al"]["survival"]
        assert np.array_equal(rec[t]["s_host"], s_prev)
        ob, olam, _ = O.size_budget(s_prev, BS, float(BS), P_SLOT)
        assert (rec[t]["b"], rec[t]["lam"]) == (ob, olam), t
        sizes.append(ob)
    assert len(set(sizes)) > 1, "the budget never changed: the loop exercised nothing"

    # the loop against the oracle, step by step with the same scalars; a near
    # tie in a selection or allocation ends the comparison (the requests'
    # paths may part there)
    ctx_o, len_o = loop.ctx.copy(), loop.ctx_len.copy()
    zeros_u, zeros_s = np.zeros((BS, 16), np.float32), np.zeros(BS, np.float32)
    compared, copied = 0, []
    for t in range(loop.steps):
        x = loop.assemble(raws[t], len_o - T0)
        o = O.step_chain(ctx_o, len_o, loop.cap, x["model_tokens"], x["model_conf_logit"], np.ones(BS, np.uint8),
                         est, rec[t]["lam"], rec[t]["b"], x["target"], np.arange(BS) * rows, zeros_u, zeros_s, 0.0,
                         5, 15, L, 256)
        g = rec[t]
        if not ok_rows(o["alloc"]["flags"]).all():
            break
        for k in ("chain_tokens", "alloc_len", "chain_src", "chain_len"):
            ref = o["alloc"]["tokens" if k == "chain_tokens" else k]
            assert np.array_equal(g["al"][k], ref), (t, k)
        assert_close(g["al"]["survival"], o["alloc"]["S"], f"survival step {t}")
        assert np.array_equal(g["out"]["out_num"], o["verify"]["out_num"]), t
        assert np.array_equal(g["out"]["out_tokens"], o["verify"]["out_tokens"]), t
        assert np.array_equal(g["ctx_len"], o["ctx_len"]), t
        copied.append(o["verify"]["out_num"][: BS // 2].mean())
        ctx_o, len_o = o["ctx"], o["ctx_len"]
        compared += 1
    assert compared >= 6, f"only {compared} steps compared"
    if compared == loop.steps:
        assert np.array_equal(ctx_g, ctx_o)
    print(f"  budgets {[r['b'] for r in rec]}, tokens per step of the copying requests "
          f"{np.round(copied, 2).tolist()}")
    assert np.mean(copied) > 6.0   # the n-gram chains of the copying requests are accepted
