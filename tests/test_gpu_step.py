"""GPU parity of the whole step (draft -> allocate -> verify -> commit) and
run-to-run bit identity."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import (assert_close, assert_rows_equal, check_verify_chain, dev, expected_commit, host,
                               ok_rows)
from workloads import synth

pytestmark = pytest.mark.gpu


def gpu_step(c, ctx, ctx_len):
    import torch
    import draft_verification_spec_amd as S
    BS = c["BS"]
    d, dl, f = S.spec_ngram_draft(ctx, ctx_len, c["n_min"], c["n_max"], 15, 256)
    al = S.spec_allocate_budget(mode="chain", model_tokens=dev(c["model_tokens"]), model_conf=dev(c["model_conf_logit"]),
                                ngram_draft=d, ngram_len=dl, ngram_feat=f, est=c["estimator"], lam=c["lam"],
                                budget=c["budget"], policy="proposed", conf_is_logit=True,
                                model_point_mass=dev(c["model_point_mass"]), ld=15)
    tgt = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, c["V"])
    out = S.spec_verify_chain(tgt, dev(np.arange(BS, dtype=np.int64) * 16), al["chain_tokens"], al["alloc_len"],
                              c["temperature"], u_accept=dev(np.ascontiguousarray(c["u_acc"][:, :15])),
                              u_sample=dev(c["u_smp"]), slot_flags=al["slot_flags"], out_flags=al["out_flags"],
                              ctx=ctx, ctx_len=ctx_len)
    torch.cuda.synchronize()
    res = dict(draft=host(d), draft_len=host(dl), feat=host(f))
    res.update({k: host(v) for k, v in al.items()})
    res.update({k: host(v) for k, v in out.items()})
    res["ctx"], res["ctx_len"] = host(ctx), host(ctx_len)
    return res


@pytest.mark.parametrize("cfg", [2, 4])
def test_full_step_matches_oracle(cfg):
    c = synth.config2(ctx_extra=64) if cfg == 2 else synth.config4(ctx_extra=64)
    print(f"step c{cfg}: BS {c['BS']} ctx {c['ctx'].shape} V {c['V']}", flush=True)
    g = gpu_step(c, dev(c["ctx"]), dev(c["ctx_len"]))
    o = O.step_chain(c["ctx"], c["ctx_len"], c["ctx"].shape[1], c["model_tokens"], c["model_conf_logit"],
                     c["model_point_mass"], c["estimator"], c["lam"], c["budget"],
                     c["target_bf16"].reshape(-1, c["V"]), np.arange(c["BS"]) * 16, c["u_acc"], c["u_smp"],
                     c["temperature"], c["n_min"], c["n_max"], 15, 256)
    assert np.array_equal(g["draft"], o["draft"]) and np.array_equal(g["feat"], o["feat"])
    ok = ok_rows(o["alloc"]["flags"])   # selection and allocation near ties
    for k in ("chain_tokens", "alloc_len", "chain_src"):
        ref = o["alloc"]["tokens" if k == "chain_tokens" else k]
        assert_rows_equal(g[k], ref, ok, k)
    assert_close(g["survival"], o["alloc"]["S"], "survival")
    full = check_verify_chain(g, o["verify"], o["alloc"]["alloc_len"], f"c{cfg} step")
    # the commit of the GPU's own emitted tokens, for every request
    ctx2, len2, fl = expected_commit(c["ctx"], c["ctx_len"], c["ctx"].shape[1], g["out_tokens"], g["out_num"])
    assert np.array_equal(g["ctx"], ctx2) and np.array_equal(g["ctx_len"], len2)
    # and for the requests whose emitted tokens are the oracle's, its own commit
    same = ~full & np.all(g["out_tokens"] == o["verify"]["out_tokens"], axis=1)
    assert_rows_equal(g["ctx"], o["ctx"], same, "ctx after commit")
    print(f"  emitted mean {o['verify']['out_num'].mean():.2f}, excused {int(full.sum())}")


def test_step_is_bit_identical_run_to_run():
    c = synth.config2(ctx_extra=64)
    a = gpu_step(c, dev(c["ctx"]), dev(c["ctx_len"]))
    b = gpu_step(c, dev(c["ctx"]), dev(c["ctx_len"]))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
