"""GPU parity: spec_verify_chain and spec_verify_tree against the oracle.

Token decisions must be bit-exact except for requests the oracle flags as
near ties; p(y), q(y) within 1e-5 relative."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import assert_rows_equal, check_verify_chain, dev, expected_commit, host
from workloads import synth

pytestmark = pytest.mark.gpu


def as_logits(x):
    """numpy fp32 or bf16 bits -> torch tensor on the GPU (bf16 kept as bf16)."""
    import torch
    if x.dtype == np.uint16:
        return synth.as_torch_bf16(x).to("cuda:0")
    return dev(x)


def verify_both(target, row_base, tokens, flags, n_slots, u_acc, u_smp, T, draft=None, drow_base=None, tag="",
                max_slots=0):
    import torch
    import draft_verification_spec_amd as S
    V = target.shape[-1]
    print(f"verify chain {tag}: bs {tokens.shape[0]} ld {tokens.shape[1]} V {V} T {T} "
          f"dtype {target.dtype} draft {draft is not None} max_slots {max_slots}", flush=True)
    g = S.spec_verify_chain(as_logits(target).reshape(-1, V), dev(row_base.astype(np.int64)), dev(tokens),
                            dev(n_slots), T, u_accept=dev(u_acc), u_sample=dev(u_smp), slot_flags=dev(flags),
                            draft_logits=None if draft is None else as_logits(draft).reshape(-1, V),
                            draft_row_base=None if draft is None else dev(drow_base.astype(np.int64)),
                            max_slots=max_slots)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    o = O.verify_chain(target.reshape(-1, V), row_base, tokens, flags, n_slots, u_acc, u_smp, T,
                       draft_logits=None if draft is None else draft.reshape(-1, V), draft_row_base=drow_base)
    check_verify_chain(g, o, n_slots, tag)
    data_bits = O.BAD_TOKEN | O.BAD_LOGITS | O.CTX_OVERFLOW
    assert np.array_equal(g["out_flags"].astype(np.uint32) & data_bits, o["flags"] & data_bits)
    assert not (g["out_flags"].astype(np.uint32) & S.FLAG_RESIDUAL_LATE).any(), "a residual sum came late"
    print(f"  accepted mean {o['out_accepted'].mean():.2f}", flush=True)
    return g, o


def test_config0_probabilistic():
    c = synth.config0()
    BS, B = c["BS"], c["B"]
    verify_both(c["target"], np.arange(BS) * (B + 1), c["tokens"], np.zeros((BS, B), np.uint8),
                np.full(BS, B, np.int32), c["u_acc"], c["u_smp"], c["temperature"], c["draft"], np.arange(BS) * B)


def test_dense_headline_bf16_probabilistic():
    """The dense verify workload at full vocabulary: bf16 target [BS, 8, V]
    and draft [BS, 7, V] rows, probabilistic slots, T = 1 (residuals drawn
    from max(0, p - q) need both rows).  BS 32 keeps the oracle to seconds."""
    c = synth.dense_headline(BS=32)
    BS, B = c["BS"], c["B"]
    verify_both(c["target_bf16"], np.arange(BS) * (B + 1), c["tokens"], np.zeros((BS, B), np.uint8),
                np.full(BS, B, np.int32), c["u_acc"], c["u_smp"], c["temperature"], c["draft_bf16"],
                np.arange(BS) * B, tag="dense bf16")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_config1_model_chain(T):
    c = synth.config1(temperature=T)
    BS, B = c["BS"], c["B"]
    verify_both(c["target"], np.arange(BS) * (B + 1), c["tokens"], np.zeros((BS, B), np.uint8),
                np.full(BS, B, np.int32), c["u_acc"], c["u_smp"], T, c["draft"], np.arange(BS) * B, tag="c1 model")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_config1_ngram_chain_point_masses(T):
    c = synth.config1()
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], 3, 3, 15, 256)
    BS = c["BS"]
    g, o = verify_both(c["ngram_target"], np.arange(BS) * 16, draft, np.full((BS, 15), 3, np.uint8), dlen,
                       c["u_acc_ng"], c["u_smp_ng"], T, tag="c1 ngram")


@pytest.mark.parametrize("cfg", [2, 4])
def test_allocated_chains_bf16(cfg):
    c = synth.config2() if cfg == 2 else synth.config4()
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], 15, 256)
    al = O.allocate_budget(c["model_tokens"], c["model_conf_logit"], True, c["model_point_mass"], draft, dlen, feat,
                           c["estimator"], c["lam"], c["budget"], "proposed", ld=15)
    BS = c["BS"]
    verify_both(c["target_bf16"], np.arange(BS) * 16, al["tokens"], al["slot_flags"], al["alloc_len"],
                c["u_acc"][:, :15], c["u_smp"], c["temperature"], tag=f"c{cfg}", max_slots=c["budget"])


def test_mixed_dtypes_and_short_grid():
    """A bf16 target with fp32 draft rows (drafts read beside their target
    chunks), and a slot bound far below the real slots (the statistics grid
    is then shorter than the work and its workgroups stride)."""
    c = synth.config0()
    BS, B = c["BS"], c["B"]
    args = (np.arange(BS) * (B + 1), c["tokens"], np.zeros((BS, B), np.uint8), np.full(BS, B, np.int32),
            c["u_acc"], c["u_smp"], c["temperature"])
    verify_both(synth.f32_to_bf16_bits(c["target"]), *args, c["draft"], np.arange(BS) * B, tag="mixed")
    verify_both(c["target"], *args, c["draft"], np.arange(BS) * B, tag="short grid", max_slots=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [20011, 4099])
def test_ragged_unaligned_and_edges(V, dtype):
    rng = np.random.Generator(np.random.Philox(1000 + V))
    BS, ld = 37, 9
    z = (rng.standard_normal((BS, ld + 1, V)) * 3).astype(np.float32)
    w = (z[:, :ld] + rng.standard_normal((BS, ld, V)).astype(np.float32)).astype(np.float32)
    y = rng.integers(0, V, (BS, ld)).astype(np.int32)
    am = np.argmax(w, -1)
    take = rng.random((BS, ld)) < 0.6
    y[take] = am[take]
    y[0, 0] = V + 5                                 # out-of-range token
    y[1, 2] = -3
    n_slots = rng.integers(0, ld + 1, BS).astype(np.int32)
    n_slots[:3] = [ld, ld, 0]
    flags = (rng.random((BS, ld)) < 0.4).astype(np.uint8)
    u_acc = rng.random((BS, ld), dtype=np.float32)
    u_smp = rng.random(BS, dtype=np.float32)
    if dtype == "bf16":
        z, w = synth.f32_to_bf16_bits(z), synth.f32_to_bf16_bits(w)
    for T in (0.0, 0.6, 1.0, 2.5):
        verify_both(z, np.arange(BS) * (ld + 1), y, flags, n_slots, u_acc, u_smp, T, w, np.arange(BS) * ld,
                    tag=f"ragged {V} {dtype}")


def test_bad_rows_are_flagged_not_read():
    import torch
    import draft_verification_spec_amd as S
    V, BS, ld = 3001, 4, 3
    rng = np.random.Generator(np.random.Philox(3))
    z = rng.standard_normal((8, V)).astype(np.float32)
    z[1, 17] = np.nan
    z[5, :] = -np.inf
    row_base = np.array([0, 4, 7, 100], np.int64)     # request 2's rows run off the end, 3 is outside
    y = np.zeros((BS, ld), np.int32)
    ua, us = rng.random((BS, ld), dtype=np.float32), rng.random(BS, dtype=np.float32)
    g = S.spec_verify_chain(dev(z), dev(row_base), dev(y), dev(np.full(BS, 2, np.int32)), 1.0,
                            u_accept=dev(ua), u_sample=dev(us))
    torch.cuda.synchronize()
    fl = host(g["out_flags"]).astype(np.uint32)
    assert np.all(fl & O.BAD_LOGITS)                 # NaN / all -inf / rows outside the buffer
    assert np.all(host(g["out_num"]) >= 1)
    # write_flags: the same flags land over whatever out_flags held
    g2 = S.spec_verify_chain(dev(z), dev(row_base), dev(y), dev(np.full(BS, 2, np.int32)), 1.0,
                             u_accept=dev(ua), u_sample=dev(us), out_flags=dev(np.full(BS, 0x5A5A5A5A, np.int32)),
                             write_flags=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(g2["out_flags"]).astype(np.uint32), fl)


def test_write_flags_equals_or_mode_on_drawn_residuals():
    """Dense probabilistic chains (residuals summed by several workgroups per
    request, drawn by the last): written flags and every output equal those
    of the OR-ed call from zero."""
    import torch
    import draft_verification_spec_amd as S
    c = synth.dense_headline(BS=16)
    BS, B, V = c["BS"], c["B"], c["V"]
    tgt = as_logits(c["target_bf16"]).reshape(-1, V)
    drf = as_logits(c["draft_bf16"]).reshape(-1, V)
    args = (tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]), dev(np.full(BS, B, np.int32)),
            c["temperature"])
    kw = dict(u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]), slot_flags=dev(np.zeros((BS, B), np.uint8)),
              draft_logits=drf, draft_row_base=dev(np.arange(BS, dtype=np.int64) * B))
    a = S.spec_verify_chain(*args, **kw)
    b = S.spec_verify_chain(*args, **kw, out_flags=dev(np.full(BS, -1, np.int32)), write_flags=True)
    torch.cuda.synchronize()
    for k in a:
        assert np.array_equal(host(a[k]), host(b[k])), k


def test_commit_appends_and_overflows():
    import torch
    import draft_verification_spec_amd as S
    c = synth.config0()
    BS, B, V = c["BS"], c["B"], c["V"]
    ctx = np.zeros((BS, 530), np.int32)
    ctx[:, :512] = c["ctx"]
    ctx_len = np.array([512, 512, 525, 512], np.int32)
    cap = np.int32(530)
    tc, tl = dev(ctx), dev(ctx_len)
    g = S.spec_verify_chain(dev(c["target"]).reshape(-1, V), dev(np.arange(BS) * (B + 1)), dev(c["tokens"]),
                            dev(np.full(BS, B, np.int32)), 1.0, u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]),
                            slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dev(c["draft"]).reshape(-1, V),
                            draft_row_base=dev(np.arange(BS) * B), ctx=tc, ctx_len=tl, ctx_cap=cap)
    torch.cuda.synchronize()
    num = host(g["out_num"])
    fl = np.zeros(BS, np.uint32)
    ref_ctx, ref_len = O.commit(ctx.copy(), ctx_len.copy(), int(cap), host(g["out_tokens"]), num, fl)
    assert np.array_equal(host(tl), ref_len) and np.array_equal(host(tc), ref_ctx)
    assert np.array_equal(host(g["out_flags"]).astype(np.uint32) & O.CTX_OVERFLOW, fl & O.CTX_OVERFLOW)
    # out of place: lengths go to a separate buffer, the inputs stay
    tc, tl, tn = dev(ctx), dev(ctx_len), dev(np.zeros(BS, np.int32))
    S.spec_verify_chain(dev(c["target"]).reshape(-1, V), dev(np.arange(BS) * (B + 1)), dev(c["tokens"]),
                        dev(np.full(BS, B, np.int32)), 1.0, u_accept=dev(c["u_acc"]), u_sample=dev(c["u_smp"]),
                        slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dev(c["draft"]).reshape(-1, V),
                        draft_row_base=dev(np.arange(BS) * B), ctx=tc, ctx_len=tl, ctx_cap=cap, ctx_len_out=tn)
    torch.cuda.synchronize()
    assert np.array_equal(host(tl), ctx_len) and np.array_equal(host(tn), ref_len)
    assert np.array_equal(host(tc), ref_ctx)


def test_tree_verify_config3():
    import torch
    import draft_verification_spec_amd as S
    c = synth.config3_inputs()
    qr, ex, el = synth.tree_queries(c["ctx"], c["ctx_len"], c["block"])
    draft, dlen, feat = O.ngram_draft(c["ctx"], c["ctx_len"], c["n_min"], c["n_max"], c["L"], 256,
                                      query_req=qr, extra=ex, extra_len=el)
    t = O.tree_build_batch(c["block"], draft, dlen, c["w_node"], c["w_none"], c["depth_max"], c["rows_cap"])
    rows = synth.tree_target_rows(3, t["node_token"], t["parent_row"], t["n_rows"], c["truth"], c["V"], c["rows_cap"])
    BS, R, V = rows.shape
    rb = np.arange(BS, dtype=np.int64) * R
    print(f"verify tree: bs {BS} rows {R} V {V}", flush=True)
    g = S.spec_verify_tree(dev(rows).reshape(-1, V), dev(rb), dev(t["node_token"]), dev(t["parent_row"]),
                           dev(t["n_rows"]))
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    o = O.verify_tree(rows.reshape(-1, V), rb, t["node_token"], t["parent_row"], t["n_rows"])
    every = np.ones(BS, bool)
    for k in ("out_tokens", "out_num", "out_path_rows", "out_argmax"):
        assert_rows_equal(g[k], o[k], every, k)
    print("  mean committed per tree:", o["out_num"].mean(), flush=True)
    # a bf16 copy of the same rows
    bits = synth.f32_to_bf16_bits(rows)
    g2 = S.spec_verify_tree(as_logits(bits).reshape(-1, V), dev(rb), dev(t["node_token"]), dev(t["parent_row"]),
                            dev(t["n_rows"]))
    torch.cuda.synchronize()
    o2 = O.verify_tree(bits.reshape(-1, V), rb, t["node_token"], t["parent_row"], t["n_rows"])
    assert_rows_equal(host(g2["out_tokens"]), o2["out_tokens"], every, "bf16 out_tokens")


@pytest.mark.parametrize("R", [64, 24])
def test_tree_verify_wide_trees_commit_and_flags(R):
    """64-row trees over fp32 rows of V 151,936 (the request's chunk partials
    no longer fit the walk's LDS stage) and 24-row trees (each row's partials
    merged by two lanes), the commit into the contexts, and the flagged
    cases: row counts outside [1, rows_max] (clamped, one of them to a single
    row), a NaN row, a context without room."""
    import torch
    import draft_verification_spec_amd as S
    rng = np.random.Generator(np.random.Philox(77 if R == 64 else 2024))
    BS, V = 12, 151936
    P, Kc, L, vocab = 15, 4, 40, 50
    block = np.stack([np.stack([rng.choice(vocab, Kc, replace=False) for _ in range(P)])
                      for _ in range(BS)]).astype(np.int32)
    ngl = rng.integers(0, L + 1, BS * (P + 1)).astype(np.int32)
    ng = rng.integers(0, vocab, (BS * (P + 1), L)).astype(np.int32)
    cm = 1 + P * Kc + (P + 1) * L
    wn = rng.standard_exponential((BS, cm)).astype(np.float32)
    wz = rng.standard_exponential((BS, cm)).astype(np.float32)
    t = O.tree_build_batch(block, ng, ngl, wn, wz, 100, R)
    nt, pr, nr = t["node_token"], t["parent_row"], t["n_rows"].copy()
    assert nr.min() == R
    # the truth follows a random root-to-leaf walk of the tree, so paths run deep
    truth = rng.integers(0, V, (BS, R + 1)).astype(np.int32)
    for r in range(BS):
        u, d = 0, 0
        while True:
            kids = [c for c in range(1, nr[r]) if pr[r, c] == u]
            if not kids or rng.random() < 0.05:
                break
            u = kids[int(rng.integers(0, len(kids)))]
            truth[r, d] = nt[r, u]
            d += 1
    rows = synth.tree_target_rows(3, nt, pr, nr, truth, V, R)
    rows[2, 0, 123] = np.nan                      # a NaN in a row every request reads
    n_in = nr.copy()
    n_in[0], n_in[1] = 0, R + 5                   # clamped to 1 and R
    n_ref = np.clip(n_in, 1, R).astype(np.int32)
    rb = np.arange(BS, dtype=np.int64) * R
    o = O.verify_tree(rows.reshape(-1, V), rb, nt, pr, n_ref)
    print(f"verify tree (wide, {R} rows): committed per tree", o["out_num"].tolist(), flush=True)
    assert o["out_num"][3:].max() > (8 if R == 64 else 4)   # best-first trees of 24 rows are shallower
    cap = 300
    ctx = rng.integers(0, V, (BS, cap)).astype(np.int32)
    ctx_len = rng.integers(0, 200, BS).astype(np.int32)
    ctx_len[3] = cap - 1                          # no room for two or more tokens
    ctx_len[4] = cap - o["out_num"][4]            # exactly enough room
    fl_ref = o["flags"].copy()
    ctx_ref, len_ref = O.commit(ctx.copy(), ctx_len.copy(), cap, o["out_tokens"], o["out_num"], fl_ref)
    tc, tl, tn = dev(ctx), dev(ctx_len), dev(np.zeros(BS, np.int32))
    g = S.spec_verify_tree(dev(rows).reshape(-1, V), dev(rb), dev(nt), dev(pr), dev(n_in), ctx=tc, ctx_len=tl,
                           ctx_cap=cap, ctx_len_out=tn)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    ok = np.ones(BS, bool)
    ok[2] = False
    for k in ("out_tokens", "out_num", "out_path_rows", "out_argmax"):
        assert_rows_equal(g[k], o[k], ok, k)
    fl = g["out_flags"].astype(np.uint32)
    BAD_LENGTH = 1 << 11
    assert fl[0] & BAD_LENGTH and fl[1] & BAD_LENGTH and not (fl[2:] & BAD_LENGTH).any()
    assert fl[2] & O.BAD_LOGITS and not (np.delete(fl, 2) & O.BAD_LOGITS).any()
    assert np.array_equal(fl & O.CTX_OVERFLOW, fl_ref & O.CTX_OVERFLOW) and fl[3] & O.CTX_OVERFLOW
    assert not fl[4] & O.CTX_OVERFLOW
    assert np.array_equal(host(tl), ctx_len)      # the input lengths stay; the new ones go to ctx_len_out
    assert np.array_equal(np.delete(host(tn), 2), np.delete(len_ref, 2))
    assert np.array_equal(np.delete(host(tc), 2, axis=0), np.delete(ctx_ref, 2, axis=0))


def test_residual_wait_fallback():
    """Dense probabilistic chains with the bounded wait for published residual
    sums set to give up at once: every request whose residual is streamed is
    flagged RESIDUAL_LATE and its drawing workgroup sums the residual itself,
    and the outputs still match the oracle (the kernel's own give-up, not a
    fault or a hang)."""
    import torch
    import draft_verification_spec_amd as S
    c = synth.dense_headline(BS=16)
    BS, B, V = c["BS"], c["B"], c["V"]
    print(f"residual wait fallback: BS {BS} V {V}", flush=True)
    tgt = as_logits(c["target_bf16"]).reshape(-1, V)
    drf = as_logits(c["draft_bf16"]).reshape(-1, V)
    g = S.spec_verify_chain(tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]),
                            dev(np.full(BS, B, np.int32)), c["temperature"], u_accept=dev(c["u_acc"]),
                            u_sample=dev(c["u_smp"]), slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=drf,
                            draft_row_base=dev(np.arange(BS, dtype=np.int64) * B), residual_wait=-1)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in g.items()}
    o = O.verify_chain(c["target_bf16"].reshape(-1, V), np.arange(BS) * (B + 1), c["tokens"],
                       np.zeros((BS, B), np.uint8), np.full(BS, B, np.int32), c["u_acc"], c["u_smp"],
                       c["temperature"], draft_logits=c["draft_bf16"].reshape(-1, V), draft_row_base=np.arange(BS) * B)
    check_verify_chain(g, o, np.full(BS, B), "residual wait fallback")
    late = (g["out_flags"].astype(np.uint32) & S.FLAG_RESIDUAL_LATE) != 0
    rejected = o["out_accepted"] < B
    assert np.array_equal(late, rejected), (late, rejected)   # exactly the streamed (rejected) requests


def test_unstaged_decide_partials():
    """32 slots of fp32 rows at V 151,936: 65 rows x 38 chunks of partials per
    request no longer fit the decide workgroup's LDS stage, so it merges them
    from global memory."""
    rng = np.random.Generator(np.random.Philox(2032))
    BS, ld, V = 3, 32, 151936
    z = (rng.standard_normal((BS, ld + 1, V)) * 2).astype(np.float32)
    w = (z[:, :ld] + 0.3 * rng.standard_normal((BS, ld, V))).astype(np.float32)
    y = np.argmax(w, -1).astype(np.int32)                 # likely accepted: long accepted runs
    n_slots = np.array([ld, ld - 5, 17], np.int32)
    u_acc = (rng.random((BS, ld)) * 0.5).astype(np.float32)
    u_smp = rng.random(BS, dtype=np.float32)
    for T in (0.0, 1.0):
        verify_both(z, np.arange(BS) * (ld + 1), y, np.zeros((BS, ld), np.uint8), n_slots, u_acc, u_smp, T, w,
                    np.arange(BS) * ld, tag="unstaged partials")


def test_large_batch_row_prefix_in_global_memory():
    """5,000 requests over rows that are not 16-byte aligned (V 4,099): the
    statistics pass keeps the row prefix in global memory."""
    rng = np.random.Generator(np.random.Philox(5000))
    BS, ld, V = 5000, 2, 4099
    z = (rng.standard_normal((BS, ld + 1, V)) * 2).astype(np.float32)
    w = (z[:, :ld] + rng.standard_normal((BS, ld, V)).astype(np.float32)).astype(np.float32)
    y = rng.integers(0, V, (BS, ld)).astype(np.int32)
    am = np.argmax(w, -1)
    take = rng.random((BS, ld)) < 0.7
    y[take] = am[take]
    n_slots = rng.integers(0, ld + 1, BS).astype(np.int32)
    flags = (rng.random((BS, ld)) < 0.3).astype(np.uint8)
    u_acc = rng.random((BS, ld), dtype=np.float32)
    u_smp = rng.random(BS, dtype=np.float32)
    verify_both(z, np.arange(BS) * (ld + 1), y, flags, n_slots, u_acc, u_smp, 1.0, w, np.arange(BS) * ld,
                tag="global row prefix")


def test_residual_over_many_chunks():
    """Rows of 2,200,000 fp32 logits (538 chunks, more than the decide
    workgroup has threads): the residual is summed chunk by chunk by the
    drawing workgroup rather than streamed."""
    rng = np.random.Generator(np.random.Philox(2200))
    BS, ld, V = 2, 1, 2200000
    z = (rng.standard_normal((BS, ld + 1, V)) * 2).astype(np.float32)
    w = (z[:, :ld] + rng.standard_normal((BS, ld, V)).astype(np.float32)).astype(np.float32)
    y = np.argmax(w, -1).astype(np.int32)
    u_acc = np.array([[0.999], [0.0]], np.float32)        # request 0 rejects (a residual), 1 accepts (a bonus)
    u_smp = rng.random(BS, dtype=np.float32)
    verify_both(z, np.arange(BS) * (ld + 1), y, np.zeros((BS, ld), np.uint8), np.full(BS, ld, np.int32), u_acc,
                u_smp, 1.0, w, np.arange(BS) * ld, tag="many chunks")
