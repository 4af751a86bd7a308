"""GPU parity of the n-gram draft fused into chain verification: after the
commit, the drawing workgroup scans each request's committed context.  Its
outputs must equal the oracle's n-gram draft over the contexts and lengths the
commit produced (bit-exact, every request), and the verification outputs must
not change when the draft is fused in."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import dev, host
from workloads import synth

pytestmark = pytest.mark.gpu


def run_pair(logits, rb, tokens, n_slots, T, ctx, ctx_len, cap, ngram, **kw):
    """The same verification with and without the fused draft, on copies of
    the contexts; returns both result dicts and the committed contexts."""
    import torch
    import draft_verification_spec_amd as S
    res = []
    for fused in (False, True):
        tc, tl, tn = dev(ctx), dev(ctx_len), dev(np.zeros(len(ctx_len), np.int32))
        out = S.spec_verify_chain(logits, rb, tokens, n_slots, T, ctx=tc, ctx_len=tl, ctx_cap=cap, ctx_len_out=tn,
                                  ngram=ngram if fused else None, **kw)
        torch.cuda.synchronize()
        r = {k: host(v) for k, v in out.items()}
        r["ctx"], r["ctx_len"] = host(tc), host(tn)
        res.append(r)
    return res


def check(plain, fused, ngram):
    n_min, n_max, L, cap = ngram
    for k, v in plain.items():
        assert np.array_equal(v, fused[k]), f"{k} changed by the fused draft"
    d, dl, f = O.ngram_draft(fused["ctx"], fused["ctx_len"], n_min, n_max, L, cap)
    assert np.array_equal(fused["ngram_len"], dl), (fused["ngram_len"], dl)
    assert np.array_equal(fused["ngram_feat"], f)
    assert np.array_equal(fused["ngram_draft"], d)
    return dl


def test_dense_headline_fused_draft():
    """The measured step: BS 128, V 151,936, bf16 rows, probabilistic slots,
    T = 1, 8,192-token contexts, n-gram n 5..15."""
    c = synth.dense_headline(ctx_extra=64)
    BS, V, B = c["BS"], c["V"], c["B"]
    print(f"dense: BS {BS} V {V} ctx {c['ctx'].shape}", flush=True)
    tgt = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, V)
    dft = synth.as_torch_bf16(c["draft_bf16"]).to("cuda:0").reshape(-1, V)
    ngram = (c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"])
    args = (tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]), dev(np.full(BS, B, np.int32)),
            c["temperature"])
    kw = dict(u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]), slot_flags=dev(np.zeros((BS, B), np.uint8)),
              draft_logits=dft, draft_row_base=dev(np.arange(BS, dtype=np.int64) * B), write_flags=True)
    ctx = c["ctx"].copy()
    plain, fused = run_pair(*args, ctx, c["ctx_len"], ctx.shape[1], ngram, **kw)
    check(plain, fused, ngram)
    # the emitted tokens are random, so the committed suffix rarely recurs;
    # plant, in every other request, an earlier copy of the last 20 tokens
    # plus the emitted ones and a continuation, then verify again (the
    # verification does not read the contexts, so it emits the same tokens)
    rng = np.random.default_rng(7)
    for r in range(0, BS, 2):
        n, L0 = plain["out_num"][r], c["ctx_len"][r]
        seq = np.concatenate([ctx[r, L0 - 20:L0], plain["out_tokens"][r, :n], rng.integers(0, V, 20)])
        ctx[r, 1000:1000 + len(seq)] = seq
    plain, fused = run_pair(*args, ctx, c["ctx_len"], ctx.shape[1], ngram, **kw)
    dl = check(plain, fused, ngram)
    assert (dl[0::2] == c["max_draft"]).all() and (fused["ngram_feat"][0::2, 2] >= 20).all()


def test_dense_draft_periodic_texts_and_full_candidate_list():
    """The dense step's fused draft on periodic texts (n_min 5).  Requests 0
    mod 4: 8,680-token texts whose body repeats the last four tokens of the
    text before the drawn token, so about 2,170 positions match four tokens
    and the candidate list (2,048) fills: the rest are extended in place.
    Requests 1 and 2 mod 4: the body repeats those four tokens and the drawn
    one, so every fifth position starts a match that runs to the comparison
    cap.  Caps 5 and 256."""
    c = synth.dense_headline(ctx_extra=64)
    BS, V, B = c["BS"], c["V"], c["B"]
    tgt = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, V)
    dft = synth.as_torch_bf16(c["draft_bf16"]).to("cuda:0").reshape(-1, V)
    args = (tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]), dev(np.full(BS, B, np.int32)),
            c["temperature"])
    kw = dict(u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]), slot_flags=dev(np.zeros((BS, B), np.uint8)),
              draft_logits=dft, draft_row_base=dev(np.arange(BS, dtype=np.int64) * B), write_flags=True)
    stride = 8704 + 16
    ctx = np.zeros((BS, stride), np.int32)
    ctx[:, :c["ctx"].shape[1]] = c["ctx"]
    lens = c["ctx_len"].astype(np.int32).copy()
    for cap in (256, 5):
        ngram = (c["n_min"], c["n_max"], c["max_draft"], cap)
        plain, _ = run_pair(*args, ctx, lens, stride, ngram, **kw)
        acc = plain["out_accepted"]
        cc, ll = ctx.copy(), lens.copy()
        for r in range(BS):
            if r % 4 == 3:
                continue   # untouched
            L0 = 8680 - int(acc[r]) if r % 4 == 0 else int(lens[r])   # long (overflow) or as generated
            text = np.concatenate([c["ctx"][r, :min(L0, c["ctx"].shape[1])], np.zeros(max(0, L0 - c["ctx"].shape[1]),
                                                                                     np.int32)])
            tail = np.concatenate([text[L0 - 4:L0], plain["out_tokens"][r, :acc[r]]])[-4:]
            y = plain["out_tokens"][r, acc[r]]
            body = np.resize(tail if r % 4 == 0 else np.concatenate([tail, [y]]), L0 - 4)
            cc[r, :L0 - 4] = body
            cc[r, L0 - 4:L0] = text[L0 - 4:L0]
            ll[r] = L0
        print(f"periodic texts: cap {cap}, {int((np.arange(BS) % 4 == 0).sum())} of 8,680 tokens", flush=True)
        plain, fused = run_pair(*args, cc, ll, stride, ngram, **kw)
        dl = check(plain, fused, ngram)
        ext = (np.arange(BS) % 4 == 1) | (np.arange(BS) % 4 == 2)
        assert (dl[ext] > 0).all(), dl


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_config0_overflow_and_long_contexts(T):
    """Commit overflow (the draft then scans the unchanged context), contexts
    longer than the scan window (three windows), ragged lengths, T = 0 and 1."""
    c = synth.config0()
    BS, B, V = c["BS"], c["B"], c["V"]
    stride = 20100
    ctx = np.zeros((BS, stride), np.int32)
    lens = np.array([20003, 511, 19995, 9000], np.int32)
    for r in range(BS):
        ctx[r] = np.resize(c["ctx"][r], stride)   # the planted text repeated: long matches
    cap = np.int32(20003)                          # request 0 is full: its commit overflows
    ngram = (3, 15, 15, 256)
    kw = dict(slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dev(c["draft"]).reshape(-1, V),
              draft_row_base=dev(np.arange(BS) * B))
    if T > 0:
        kw.update(u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]))
    plain, fused = run_pair(dev(c["target"]).reshape(-1, V), dev(np.arange(BS) * (B + 1)), dev(c["tokens"]),
                            dev(np.full(BS, B, np.int32)), T, ctx, lens, cap, ngram, **kw)
    check(plain, fused, ngram)
    over = (plain["out_flags"].astype(np.uint32) & O.CTX_OVERFLOW) != 0
    assert over.any() and np.array_equal(fused["ctx_len"][over], lens[over])
    # n_min 5 and the same texts (one decide workgroup per request at this
    # vocabulary)
    ngram5 = (5, 15, 15, 256)
    plain, fused = run_pair(dev(c["target"]).reshape(-1, V), dev(np.arange(BS) * (B + 1)), dev(c["tokens"]),
                            dev(np.full(BS, B, np.int32)), T, ctx, lens, cap, ngram5, **kw)
    check(plain, fused, ngram5)


def test_point_mass_chain_fused_draft():
    """Point-mass slots (the residual is p without y) and all-accepted bonus
    draws, fp32 rows at full vocabulary, n = 4."""
    c = synth.config1()
    BS, V = c["BS"], c["V"]
    ng = O.ngram_draft(c["ctx"], c["ctx_len"], 4, 4, 15, 256)
    toks = np.where(ng[0] >= 0, ng[0], 0).astype(np.int32)
    stride = c["ctx"].shape[1] + 32
    ctx = np.zeros((BS, stride), np.int32)
    ctx[:, :c["ctx"].shape[1]] = c["ctx"]
    ngram = (4, 4, 15, 256)
    plain, fused = run_pair(dev(c["ngram_target"]).reshape(-1, V), dev(np.arange(BS) * 16), dev(toks),
                            dev(ng[1]), 1.0, ctx, c["ctx_len"], stride, ngram, u_accept=dev(c["u_acc_ng"]),
                            u_sample=dev(c["u_smp_ng"]), slot_flags=dev(np.ones((BS, 15), np.uint8)))
    check(plain, fused, ngram)


def test_measured_step_call_matches_oracle():
    """The reported step exactly as it is timed: one call with uniforms drawn
    in the kernel (Philox4x32-10, seed 20261202, step 1), the acceptance
    histogram, written flags, the commit into the contexts with new lengths
    apart, and the next n-gram draft fused in.  Its verification outputs
    against the oracle's with the oracle's own uniforms; the contexts against
    the commit of the emitted tokens; the draft against the oracle's scan of
    the committed contexts; the histogram against the accepted counts."""
    import torch
    import draft_verification_spec_amd as S
    from tests.gpu_helpers import check_verify_chain, expected_commit
    seed, step = 20261202, 1
    c = synth.dense_headline(ctx_extra=64)
    BS, V, B = c["BS"], c["V"], c["B"]
    print(f"measured step call: BS {BS} V {V} B {B}", flush=True)
    tgt = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, V)
    dft = synth.as_torch_bf16(c["draft_bf16"]).to("cuda:0").reshape(-1, V)
    ctx, ctx_len = dev(c["ctx"]), dev(c["ctx_len"])
    ctx_len_new = torch.empty_like(ctx_len)
    hist = torch.zeros(B + 1, dtype=torch.int32, device="cuda:0")
    out = S.spec_verify_chain(tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]),
                              dev(np.full(BS, B, np.int32)), c["temperature"], rng=(seed, step), accept_hist=hist,
                              slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dft,
                              draft_row_base=dev(np.arange(BS, dtype=np.int64) * B), ctx=ctx, ctx_len=ctx_len,
                              ctx_len_out=ctx_len_new, write_flags=True,
                              ngram=(c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"]))
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    u_acc, u_smp = O.step_uniforms(BS, B, seed, step)
    ref = O.verify_chain(c["target_bf16"].reshape(-1, V), np.arange(BS) * (B + 1), c["tokens"],
                         np.zeros((BS, B), np.uint8), np.full(BS, B, np.int32), u_acc, u_smp, c["temperature"],
                         draft_logits=c["draft_bf16"].reshape(-1, V), draft_row_base=np.arange(BS) * B)
    check_verify_chain(g, ref, np.full(BS, B), "measured step")
    c2, l2, _ = expected_commit(c["ctx"], c["ctx_len"], c["ctx"].shape[1], g["out_tokens"], g["out_num"])
    assert np.array_equal(host(ctx), c2) and np.array_equal(host(ctx_len_new), l2)
    assert np.array_equal(host(ctx_len), c["ctx_len"])   # the old lengths are left as they were
    d, dl, f = O.ngram_draft(c2, l2, c["n_min"], c["n_max"], c["max_draft"], c["copy_cap"])
    assert np.array_equal(g["ngram_len"], dl) and np.array_equal(g["ngram_feat"], f)
    assert np.array_equal(g["ngram_draft"], d)
    assert np.array_equal(host(hist), np.bincount(g["out_accepted"], minlength=B + 1))
