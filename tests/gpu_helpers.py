"""Helpers shared by the GPU parity tests (comparison rules, device copies)."""
import numpy as np

from oracle import oracle as O

# Requests whose decisions before the final draw the oracle flags as near ties
# (an accept test, a chain selection, an allocation cut or a tree order), or
# whose residual had no mass, are excused from bit-exact comparison of their
# tokens.  A near tie of the final draw alone (SAMPLE_NEAR) excuses only that
# token: it must lie in the oracle's tie window, and everything before it is
# compared exactly.
EXCUSE = O.ACCEPT_NEAR | O.SELECT_NEAR | O.ALLOC_NEAR | O.TREE_NEAR | O.RESIDUAL_ZERO
RTOL = 1e-5          # probabilities / survivals / Q, relative, fp32
ATOL = 1e-37         # below the smallest normal fp32


def dev(a, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def ok_rows(flags):
    return (np.asarray(flags).astype(np.uint32) & EXCUSE) == 0


def assert_rows_equal(gpu, ref, ok, name):
    gpu, ref = np.asarray(gpu), np.asarray(ref)
    bad = [r for r in range(len(ref)) if ok[r] and not np.array_equal(gpu[r], ref[r])]
    assert not bad, f"{name}: {len(bad)} requests differ, first {bad[:5]}: gpu={gpu[bad[0]]} ref={ref[bad[0]]}"


def assert_close(gpu, ref, name, rtol=RTOL, atol=ATOL, mask=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref) - (rtol * np.abs(ref) + atol)
    if mask is not None:
        err = np.where(mask, err, -1.0)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= 0, \
        f"{name}: |gpu-ref| beyond {rtol} rel at {worst}: gpu={gpu[worst]!r} ref={ref[worst]!r}"


def excused_fraction(flags):
    return float(np.mean(~ok_rows(flags)))


def check_verify_chain(g, o, n_slots, tag=""):
    """Chain verification outputs g (GPU, numpy) against the oracle's o.

    Every request not excused by EXCUSE must agree on its accepted count,
    out_num and accepted tokens; its final token must equal the oracle's, or
    for a SAMPLE_NEAR request lie in the oracle's tie window [win_lo, win_hi];
    the padding after it is -1.  p(y), q(y) of every slot within RTOL, and p
    of the bonus row (column n_slots) wherever the final token is the
    oracle's.  Returns the mask of fully excused requests."""
    fl = np.asarray(o["flags"]).astype(np.uint32)
    full = (fl & EXCUSE) != 0
    near = ~full & ((fl & O.SAMPLE_NEAR) != 0)
    exact = ~full & ~near
    assert_rows_equal(g["out_accepted"], o["out_accepted"], ~full, "out_accepted")
    assert_rows_equal(g["out_num"], o["out_num"], ~full, "out_num")
    assert_rows_equal(g["out_tokens"], o["out_tokens"], exact, "out_tokens")
    gt_all = np.asarray(g["out_tokens"])
    same_last = exact.copy()
    moved = 0
    for r in np.nonzero(near)[0]:
        n = int(o["out_accepted"][r])
        gt = gt_all[r]
        assert np.array_equal(gt[:n], o["out_tokens"][r, :n]), f"request {r}: accepted tokens differ"
        assert np.all(gt[n + 1:] == -1), f"request {r}: padding after the final token"
        tok = int(gt[n])
        assert o["win_lo"][r] <= tok <= o["win_hi"][r], \
            f"request {r}: drawn token {tok} outside the tie window [{o['win_lo'][r]}, {o['win_hi'][r]}]"
        same_last[r] = tok == o["out_tokens"][r, n]
        moved += not same_last[r]
    assert_close(g["out_q"], o["out_q"], "q(y)")
    gp = np.asarray(g["out_p"])
    ld = gp.shape[1] - 1
    mask = np.ones(gp.shape, bool)
    b = np.clip(np.asarray(n_slots), 0, ld)
    for r in np.nonzero(~same_last)[0]:
        mask[r, b[r]] = False   # the bonus row's p is read at the drawn token
    assert_close(gp, o["out_p"], "p(y)", mask=mask)
    print(f"  {tag}: {int(exact.sum())} requests exact, {int(near.sum())} with the draw in its tie window "
          f"({moved} of them another token of the window), {int(full.sum())} excused", flush=True)
    return full


def expected_commit(ctx, ctx_len, cap, out_tokens, out_num):
    """The oracle's commit of the GPU's own emitted tokens: (contexts, lengths, overflow flags)."""
    fl = np.zeros(len(ctx_len), np.uint32)
    c2, l2 = O.commit(np.array(ctx, np.int32, copy=True), np.array(ctx_len, np.int32, copy=True), int(cap),
                      np.asarray(out_tokens), np.asarray(out_num), fl)
    return c2, l2, fl
