"""NumPy front end of the C oracle (``spec_oracle.c``).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It never imports the
HIP package and the HIP package never imports it.

The functions take and return NumPy arrays; all arithmetic happens in the C
library in fp64.  ``step_chain`` and ``tree_step`` compose the per-request
steps in the order the pages give them (scan, estimate, select, allocate,
verify, commit).
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "spec_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# flag bits (same meanings as the library's per-request out_flags)
ACCEPT_NEAR, SAMPLE_NEAR, SELECT_NEAR, ALLOC_NEAR, TREE_NEAR, RESIDUAL_ZERO = (1 << i for i in range(6))
BAD_TOKEN, BAD_LOGITS, CTX_OVERFLOW, BAD_LENGTH, BAD_FOREST = 1 << 8, 1 << 9, 1 << 10, 1 << 11, 1 << 13
NEAR_MASK = ACCEPT_NEAR | SAMPLE_NEAR | SELECT_NEAR | ALLOC_NEAR | TREE_NEAR
SLOT_POINT_MASS, SLOT_FROM_NGRAM = 1, 2
POLICIES = {"proposed": 0, "ngram_first": 1, "extension": 2, "model_only": 3, "ngram_only": 4}


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC",
                               "-o", LIB, SRC, "-lm"])
    return LIB


_lib = None


def _load(path):
    h = C.CDLL(path)
    h.oracle_estimate_logit.restype = C.c_double
    h.oracle_chain_value.restype = C.c_double
    h.oracle_select.restype = C.c_int
    h.oracle_tree_build.restype = C.c_int
    h.oracle_tree_forest.restype = C.c_int
    h.oracle_size_budget.restype = C.c_int
    h.oracle_step_cost.restype = C.c_double
    return h


def lib():
    global _lib
    if _lib is None:
        _lib = _load(build())
    return _lib


def build_mutant(path: str, mutation: int) -> str:
    """Compile the oracle with a planted mistake (see SPEC_ORACLE_MUTATION)."""
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC",
                           f"-DSPEC_ORACLE_MUTATION={int(mutation)}", "-o", path, SRC, "-lm"])
    return path


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every call through another build of the oracle."""
    global _lib
    old = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = old


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


class _Est(C.Structure):
    _fields_ = [("beta", C.c_double * 15)] + [(n, C.c_double) for n in (
        "w_first", "w_rest", "delta", "l_first", "l_rest", "k_first", "k_rest",
        "n_ref", "n_full", "m_ref", "m_cap")]


def _est(e) -> _Est:
    s = _Est()
    for i in range(15):
        s.beta[i] = float(np.float32(e.beta[i]))
    for n in ("w_first", "w_rest", "delta", "l_first", "l_rest", "k_first", "k_rest",
              "n_ref", "n_full", "m_ref", "m_cap"):
        setattr(s, n, float(getattr(e, n)))
    return s


# ---------------------------------------------------------------------------
# n-gram draft
# ---------------------------------------------------------------------------

def ngram_draft(ctx, ctx_len, n_min, n_max, max_draft=15, copy_cap=256,
                query_req=None, extra=None, extra_len=None, follow_ctx=0):
    """Returns (draft, draft_len, feat), and with follow_ctx > 0 (the tree's
    n-gram fill with its follower fallback) also the follower counts."""
    ctx = _c(ctx, np.int32)
    ctx_len = _c(ctx_len, np.int32)
    nq = len(query_req) if query_req is not None else ctx.shape[0]
    qr = None if query_req is None else _c(query_req, np.int32)
    ex = None if extra is None else _c(extra, np.int32)
    el = None if extra_len is None else _c(extra_len, np.int32)
    draft = np.full((nq, max_draft), -1, np.int32)
    dlen = np.zeros(nq, np.int32)
    feat = np.zeros((nq, 4), np.int32)
    follow = np.zeros((nq, max_draft), np.int32)
    lib().oracle_ngram_draft(C.c_int(nq), _p(ctx), C.c_int64(ctx.shape[1]), _p(ctx_len), _p(qr), _p(ex),
                             C.c_int64(0 if ex is None else ex.shape[1]), _p(el),
                             C.c_int(n_min), C.c_int(n_max), C.c_int(max_draft), C.c_int(copy_cap),
                             C.c_int(follow_ctx), _p(draft), _p(dlen), _p(feat), _p(follow))
    if follow_ctx > 0:
        return draft, dlen, feat, follow
    return draft, dlen, feat


# ---------------------------------------------------------------------------
# estimator, survivals, selection, allocation
# ---------------------------------------------------------------------------

def estimate_logit(est, k, n, a, m) -> float:
    e = _est(est)
    return lib().oracle_estimate_logit(C.byref(e), C.c_int(k), C.c_int(n), C.c_int(a), C.c_int(m))


def estimate(est, n, a, m, length) -> np.ndarray:
    e = _est(est)
    h = np.zeros(max(length, 1), np.float64)
    lib().oracle_estimate(C.byref(e), C.c_int(n), C.c_int(a), C.c_int(m), C.c_int(length), _p(h))
    return h[:length]


def survival(alpha) -> np.ndarray:
    a = _c(alpha, np.float64)
    S = np.zeros(max(len(a), 1), np.float64)
    lib().oracle_survival(_p(a), C.c_int(len(a)), _p(S))
    return S[:len(a)]


def chain_value(S, lam) -> float:
    S = _c(S, np.float64)
    return lib().oracle_chain_value(_p(S), C.c_int(len(S)), C.c_double(lam))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def select(d, c, g, h, lam, policy="proposed", model_point_mass=True, K=None, ld=15):
    d = _c(d, np.int32)
    c = _c(c, np.float64)
    g = _c(g, np.int32) if len(g) else np.zeros(1, np.int32)
    glen = len(h)
    h = _c(h, np.float64) if glen else np.zeros(1, np.float64)
    K = len(d) if K is None else K
    tok = np.full(ld, -1, np.int32)
    fl = np.zeros(ld, np.uint8)
    S = np.zeros(ld, np.float64)
    src = C.c_int32(0)
    near = C.c_int(0)
    n = lib().oracle_select(C.c_int(K), _p(d), _p(c), C.c_int(len(d)), _p(g), _p(h), C.c_int(glen),
                            C.c_double(lam), C.c_int(POLICIES[policy]), C.c_int(int(model_point_mass)),
                            C.c_int(ld), _p(tok), _p(fl), _p(S), C.byref(src), C.byref(near))
    return dict(tokens=tok, flags=fl, S=S, len=n, src=src.value, near=bool(near.value))


class _Cost(C.Structure):
    _fields_ = [("c0", C.c_double), ("p", C.c_double), ("graph_limit", C.c_int32), ("n_tokens", C.c_int32),
                ("eager", C.c_void_p), ("n_eager", C.c_int32)]


def _cost(c0, p, graph_limit=0, n_tokens=0, eager=None):
    eg = None if eager is None else _c(eager, np.float64)
    cm = _Cost(float(c0), float(p), int(graph_limit), int(n_tokens), _p(eg), 0 if eg is None else len(eg))
    return cm, eg   # keep the table alive with the struct


def step_cost(b, c0, p, graph_limit=0, n_tokens=0, eager=None):
    """C(b) of the cost model ([HS] Appendix F, Eq. (4)), or a negative value when b cannot run."""
    cm, keep = _cost(c0, p, graph_limit, n_tokens, eager)
    lib().oracle_step_cost.restype = C.c_double
    return lib().oracle_step_cost(C.byref(cm), C.c_int(int(b)))


def size_budget(S, n_requests, c0, p, b_max=None, graph_limit=0, n_tokens=0, eager=None):
    """Budget sizing ([HS] Section 2 and Section 4.3 Eq. (2)): returns (b*, lambda, G[0..b_max])."""
    S = _c(np.ravel(S), np.float32)
    n = len(S)
    b_max = n if b_max is None else int(b_max)
    G = np.zeros(min(b_max, n) + 1, np.float64)
    lam = C.c_double(0.0)
    cm, keep = _cost(c0, p, graph_limit, n_tokens, eager)
    b = lib().oracle_size_budget(_p(S), C.c_int(n), C.c_int(int(n_requests)), C.byref(cm), C.c_int(b_max), _p(G),
                                 C.byref(lam))
    return b, lam.value, G


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon et al., SC'11) of a 4-word counter and 2-word key."""
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def philox4x64_10(ctr, key):
    """Philox4x64-10, the 64-bit member of the same family."""
    c = _c(ctr, np.uint64)
    k = _c(key, np.uint64)
    out = np.zeros(4, np.uint64)
    lib().oracle_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def step_uniforms(bs, ld, seed, offset):
    """The uniforms a verification step draws for itself: (u_accept [bs, ld], u_sample [bs])."""
    u_acc = np.zeros((bs, ld), np.float32)
    u_smp = np.zeros(bs, np.float32)
    lib().oracle_step_uniforms(C.c_int(bs), C.c_int(ld), C.c_uint64(int(seed)), C.c_uint64(int(offset)),
                               _p(u_acc), _p(u_smp))
    return u_acc, u_smp


def stale_shortfall(sigma, n_requests):
    """Eq. (5) of [HS] Appendix O: the mean shortfall of a stale budget on the
    steps where it is too small, E[-D | D < 0] = sqrt(2/pi) sigma sqrt(B), for a
    batch miscount D that is normal with standard deviation sigma sqrt(B)."""
    return np.sqrt(2.0 / np.pi) * sigma * np.sqrt(n_requests)


def allocate(lens, S, budget, flags=None):
    lens = _c(lens, np.int32)
    S = _c(S, np.float64)
    bs, ld = S.shape
    alloc = np.zeros(bs, np.int32)
    row_base = np.zeros(bs, np.int64)
    total = C.c_int32(0)
    fl = np.zeros(bs, np.uint32) if flags is None else flags
    lib().oracle_allocate(C.c_int(bs), C.c_int(ld), _p(lens), _p(S), C.c_int(budget),
                          _p(alloc), _p(row_base), C.byref(total), _p(fl))
    return alloc, row_base, total.value, fl


def allocate_budget(model_tokens, model_conf, conf_is_logit, model_point_mass, ng_draft, ng_len, ng_feat,
                    est, lam, budget, policy="proposed", ld=15):
    """Per request: estimate h from the scan's features, survivals, select one
    chain; then allocate the batch budget over the chosen chains."""
    bs, K = model_tokens.shape
    conf = np.asarray(model_conf, np.float64)
    c_all = sigmoid(conf) if conf_is_logit else conf
    out = dict(tokens=np.full((bs, ld), -1, np.int32), slot_flags=np.zeros((bs, ld), np.uint8),
               S=np.zeros((bs, ld), np.float64), chain_len=np.zeros(bs, np.int32),
               chain_src=np.zeros(bs, np.int32), h=np.zeros((bs, ld), np.float64),
               flags=np.zeros(bs, np.uint32))
    for r in range(bs):
        glen = int(ng_len[r])
        n, a, m = (int(v) for v in ng_feat[r, :3])
        h = estimate(est, n, a, m, glen) if glen else np.zeros(0)
        out["h"][r, :glen] = h
        sel = select(model_tokens[r], c_all[r], ng_draft[r, :glen], h, lam, policy,
                     bool(model_point_mass[r]), K=K, ld=ld)
        out["tokens"][r] = sel["tokens"]
        out["slot_flags"][r] = sel["flags"]
        out["S"][r] = sel["S"]
        out["chain_len"][r] = sel["len"]
        out["chain_src"][r] = sel["src"]
        if sel["near"]:
            out["flags"][r] |= SELECT_NEAR
    alloc, row_base, total, fl = allocate(out["chain_len"], out["S"], budget, out["flags"])
    out.update(alloc_len=alloc, row_base=row_base, total_rows=total, flags=fl)
    return out


# ---------------------------------------------------------------------------
# verification
# ---------------------------------------------------------------------------

def _logits(x):
    """Accept fp32 arrays or uint16 bf16 bit patterns; returns (array, dtype code)."""
    if x is None:
        return None, 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    return np.ascontiguousarray(x, dtype=np.float32), 0


def verify_chain(logits, row_base, tokens, slot_flags, n_slots, u_acc, u_smp, temperature,
                 draft_logits=None, draft_row_base=None, flags=None):
    """logits: [rows, V] (fp32 or bf16 bits); tokens/slot_flags/u_acc: [bs, ld].

    Returns out_tokens [bs, ld+1], out_num, out_accepted, out_p [bs, ld+1]
    (p(y) per slot, then p of the bonus row at the bonus token), out_q
    [bs, ld], flags, and the final draw's tie window [win_lo, win_hi]: the
    tokens whose CDF interval meets the band of 1e-6 W around u'W (the drawn
    token alone unless the request is flagged SAMPLE_NEAR)."""
    lg, dt = _logits(logits)
    dl, ddt = _logits(draft_logits)
    V = lg.shape[-1]
    lg2 = lg.reshape(-1, V)
    dl2 = None if dl is None else dl.reshape(-1, V)
    tokens = _c(tokens, np.int32)
    bs, ld = tokens.shape
    slot_flags = _c(slot_flags, np.uint8)
    n_slots = _c(n_slots, np.int32)
    u_acc = _c(u_acc, np.float32)
    u_smp = _c(u_smp, np.float32)
    row_base = _c(row_base, np.int64)
    drb = None if draft_row_base is None else _c(draft_row_base, np.int64)
    out_tokens = np.full((bs, ld + 1), -1, np.int32)
    out_num = np.zeros(bs, np.int32)
    out_acc = np.zeros(bs, np.int32)
    out_p = np.zeros((bs, ld + 1), np.float64)
    out_q = np.zeros((bs, ld), np.float64)
    win_lo = np.zeros(bs, np.int32)
    win_hi = np.zeros(bs, np.int32)
    fl = np.zeros(bs, np.uint32) if flags is None else flags.astype(np.uint32).copy()
    lib().oracle_verify_chain(C.c_int(bs), C.c_int(V), C.c_double(temperature),
                              _p(lg2), C.c_int(dt), C.c_int64(V), _p(row_base),
                              _p(dl2), C.c_int(ddt), C.c_int64(V), _p(drb),
                              _p(tokens), _p(slot_flags), C.c_int(ld), _p(n_slots), _p(u_acc), _p(u_smp),
                              _p(out_tokens), _p(out_num), _p(out_acc), _p(out_p), _p(out_q), _p(fl),
                              _p(win_lo), _p(win_hi))
    return dict(out_tokens=out_tokens, out_num=out_num, out_accepted=out_acc, out_p=out_p, out_q=out_q,
                flags=fl, win_lo=win_lo, win_hi=win_hi)


def commit(ctx, ctx_len, ctx_cap, out_tokens, out_num, flags):
    ctx = np.ascontiguousarray(ctx, np.int32)
    ctx_len = np.ascontiguousarray(ctx_len, np.int32)
    out_tokens = _c(out_tokens, np.int32)
    out_num = _c(out_num, np.int32)
    lib().oracle_commit(C.c_int(ctx.shape[0]), _p(ctx), C.c_int64(ctx.shape[1]), _p(ctx_len),
                        C.c_int(ctx_cap), _p(out_tokens), C.c_int(out_tokens.shape[1]), _p(out_num), _p(flags))
    return ctx, ctx_len


# ---------------------------------------------------------------------------
# trees
# ---------------------------------------------------------------------------

class _TreeScore(C.Structure):
    _fields_ = [("a", C.c_double * 7), ("w_bucket", C.c_double * 64), ("w_agreed", (C.c_double * 2) * 64),
                ("w_contra", (C.c_double * 2) * 8), ("psi_depth", C.c_double * 16), ("h", C.c_void_p),
                ("sigma", C.c_void_p), ("r_share", C.c_void_p), ("psi_ctx", C.c_double), ("b_req", C.c_double),
                ("p_src", C.c_double), ("ng_feat", C.c_void_p)]


def tree_score_struct(coef, h, sigma, r_share, psi_ctx, b_req, p_src, ng_feat):
    """Eq. (6) scoring inputs of one request: coef holds a [7], w_bucket [64],
    w_agreed [64, 2], w_contra [8, 2], psi_depth [16]; h, sigma [P]; r_share
    [P, Kc]; ng_feat [P + 1, 4].  Returns (struct, arrays it points to)."""
    keep = [_c(h, np.float64), _c(sigma, np.float64), _c(r_share, np.float64), _c(ng_feat, np.int32)]
    st = _TreeScore()
    st.a[:] = [float(x) for x in coef["a"]]
    st.w_bucket[:] = [float(x) for x in coef["w_bucket"]]
    for i in range(64):
        st.w_agreed[i][:] = [float(x) for x in coef["w_agreed"][i]]
    for i in range(8):
        st.w_contra[i][:] = [float(x) for x in coef["w_contra"][i]]
    st.psi_depth[:] = [float(x) for x in coef["psi_depth"]]
    st.h, st.sigma, st.r_share, st.ng_feat = (_p(a) for a in keep)
    st.psi_ctx, st.b_req, st.p_src = float(psi_ctx), float(b_req), float(p_src)
    return st, keep


def tree_build(block, ng_draft, ng_len, w_node=None, w_none=None, depth_max=32, rows_cap=16, scores=None,
               c_max=None, ng_follow=None):
    """block: [P, Kc]; ng_draft: [P+1, L]; returns the verify rows, the S(n)
    curve and the forest.  Weights by candidate index (w_node, w_none), or the
    Eq. (6) scores (``scores``: the keyword arguments of tree_score_struct).
    ng_follow [P+1, L]: follower counts of the chains' tokens (0 = copied)."""
    block = _c(block, np.int32)
    P, Kc = block.shape
    ng = _c(ng_draft, np.int32)
    L = ng.shape[1]
    ngl = _c(ng_len, np.int32)
    nf = None if ng_follow is None else _c(ng_follow, np.int32)
    wn = None if w_node is None else _c(w_node, np.float32)
    wz = None if w_none is None else _c(w_none, np.float32)
    c_max = len(wn) if c_max is None else int(c_max)
    sc, keep = (None, None) if scores is None else tree_score_struct(**scores)
    S_curve = np.zeros(rows_cap, np.float64)
    node_token = np.full(rows_cap, -1, np.int32)
    parent_row = np.full(rows_cap, -1, np.int32)
    Q = np.zeros(rows_cap, np.float64)
    n_rows = C.c_int32(0)
    ft = np.zeros(c_max, np.int32)
    fp = np.zeros(c_max, np.int32)
    fk = np.zeros(c_max, np.int32)
    fQ = np.zeros(c_max, np.float64)
    flag = C.c_uint32(0)
    cnt = lib().oracle_tree_build(C.c_int(P), C.c_int(Kc), _p(block), C.c_int(L), _p(ng), _p(ngl), _p(nf),
                                  _p(wn), _p(wz), C.c_int(c_max), C.c_int(depth_max), C.c_int(rows_cap),
                                  None if sc is None else C.byref(sc),
                                  _p(node_token), _p(parent_row), _p(Q), C.byref(n_rows), _p(S_curve),
                                  _p(ft), _p(fp), _p(fk), _p(fQ), C.byref(flag))
    return dict(node_token=node_token, parent_row=parent_row, Q=Q, n_rows=n_rows.value, count=cnt,
                S_curve=S_curve, f_token=ft[:cnt], f_parent=fp[:cnt], f_kind=fk[:cnt], f_Q=fQ[:cnt],
                flag=flag.value)


def tree_build_batch(block, ng_draft, ng_len, w_node=None, w_none=None, depth_max=32, rows_cap=16, scores=None,
                     c_max=None, ng_follow=None):
    """block [BS,P,Kc], ng_draft [BS*(P+1), L], ng_len [BS*(P+1)], weights [BS, c_max], or ``scores``:
    a list of per-request keyword dicts of tree_score_struct; ng_follow [BS*(P+1), L] or None."""
    BS, P, _ = block.shape
    L = ng_draft.shape[1]
    ng = ng_draft.reshape(BS, P + 1, L)
    ngl = ng_len.reshape(BS, P + 1)
    nf = None if ng_follow is None else np.asarray(ng_follow).reshape(BS, P + 1, L)
    out = dict(node_token=np.full((BS, rows_cap), -1, np.int32), parent_row=np.full((BS, rows_cap), -1, np.int32),
               Q=np.zeros((BS, rows_cap)), n_rows=np.zeros(BS, np.int32), count=np.zeros(BS, np.int32),
               flags=np.zeros(BS, np.uint32), S_curve=np.zeros((BS, rows_cap)), forests=[])
    for r in range(BS):
        f = None if nf is None else nf[r]
        if scores is None:
            t = tree_build(block[r], ng[r], ngl[r], w_node[r], w_none[r], depth_max, rows_cap, ng_follow=f)
        else:
            t = tree_build(block[r], ng[r], ngl[r], None, None, depth_max, rows_cap, scores=scores[r], c_max=c_max,
                           ng_follow=f)
        out["S_curve"][r] = t["S_curve"]
        for k in ("node_token", "parent_row", "Q"):
            out[k][r] = t[k]
        out["n_rows"][r] = t["n_rows"]
        out["count"][r] = t["count"]
        out["flags"][r] = t["flag"]
        out["forests"].append(t)
    out["row_base"] = np.concatenate([[0], np.cumsum(out["n_rows"])[:-1]]).astype(np.int64)
    return out


def tree_forest(token, parent, q, n, rows_cap=16):
    """Rows from a caller-built forest of one request: token, parent [c_max]
    (node 0 = the anchor), q [c_max] fp32 acceptance estimates given the
    parent, n nodes incl. the anchor.  Returns the verify rows, the S(n)
    curve, the path products and the flags."""
    token = _c(token, np.int32)
    parent = _c(parent, np.int32)
    q = _c(q, np.float32)
    c_max = len(token)
    node_token = np.full(rows_cap, -1, np.int32)
    parent_row = np.full(rows_cap, -1, np.int32)
    Q = np.zeros(rows_cap, np.float64)
    S_curve = np.zeros(rows_cap, np.float64)
    fQ = np.zeros(c_max, np.float64)
    n_rows = C.c_int32(0)
    flag = C.c_uint32(0)
    used = lib().oracle_tree_forest(C.c_int(int(n)), C.c_int(c_max), _p(token), _p(parent), _p(q), C.c_int(rows_cap),
                                    _p(node_token), _p(parent_row), _p(Q), C.byref(n_rows), _p(S_curve), _p(fQ),
                                    C.byref(flag))
    return dict(node_token=node_token, parent_row=parent_row, Q=Q, n_rows=n_rows.value, count=used,
                S_curve=S_curve, f_Q=fQ[:used], flag=flag.value)


def tree_forest_batch(token, parent, q, n, rows_cap=16):
    """token, parent, q [BS, c_max]; n [BS]."""
    BS = token.shape[0]
    out = dict(node_token=np.full((BS, rows_cap), -1, np.int32), parent_row=np.full((BS, rows_cap), -1, np.int32),
               Q=np.zeros((BS, rows_cap)), n_rows=np.zeros(BS, np.int32), count=np.zeros(BS, np.int32),
               flags=np.zeros(BS, np.uint32), S_curve=np.zeros((BS, rows_cap)))
    for r in range(BS):
        t = tree_forest(token[r], parent[r], q[r], n[r], rows_cap)
        for k in ("node_token", "parent_row", "Q", "S_curve"):
            out[k][r] = t[k]
        out["n_rows"][r] = t["n_rows"]
        out["count"][r] = t["count"]
        out["flags"][r] = t["flag"]
    out["row_base"] = np.concatenate([[0], np.cumsum(out["n_rows"])[:-1]]).astype(np.int64)
    return out


def verify_tree(logits, row_base, node_token, parent_row, n_rows, flags=None):
    lg, dt = _logits(logits)
    V = lg.shape[-1]
    lg2 = lg.reshape(-1, V)
    node_token = _c(node_token, np.int32)
    bs, rows_max = node_token.shape
    parent_row = _c(parent_row, np.int32)
    n_rows = _c(n_rows, np.int32)
    row_base = _c(row_base, np.int64)
    out_tokens = np.full((bs, rows_max), -1, np.int32)
    out_num = np.zeros(bs, np.int32)
    out_path = np.full((bs, rows_max), -1, np.int32)
    out_arg = np.full((bs, rows_max), -1, np.int32)
    fl = np.zeros(bs, np.uint32) if flags is None else flags.astype(np.uint32).copy()
    lib().oracle_verify_tree(C.c_int(bs), C.c_int(V), _p(lg2), C.c_int(dt), C.c_int64(V), _p(row_base),
                             _p(node_token), _p(parent_row), _p(n_rows), C.c_int(rows_max),
                             _p(out_tokens), _p(out_num), _p(out_path), _p(out_arg), _p(fl))
    return dict(out_tokens=out_tokens, out_num=out_num, out_path_rows=out_path, out_argmax=out_arg, flags=fl)


# ---------------------------------------------------------------------------
# the composed chain step (draft -> allocate -> verify -> commit)
# ---------------------------------------------------------------------------

def step_chain(ctx, ctx_len, ctx_cap, model_tokens, model_conf_logit, model_point_mass, est, lam, budget,
               target, target_row_base, u_acc, u_smp, temperature, n_min=5, n_max=15, max_draft=15,
               copy_cap=256, policy="proposed", ld=15):
    """One whole step over a batch.  ``target``: [rows, V] with request r's row
    k at ``target_row_base[r] + k``.  Returns every intermediate result."""
    draft, dlen, feat = ngram_draft(ctx, ctx_len, n_min, n_max, max_draft, copy_cap)
    al = allocate_budget(model_tokens, model_conf_logit, True, model_point_mass, draft, dlen, feat, est,
                         lam, budget, policy, ld)
    ver = verify_chain(target, target_row_base, al["tokens"], al["slot_flags"], al["alloc_len"],
                       u_acc[:, :ld], u_smp, temperature, flags=al["flags"])
    ctx2, len2 = commit(ctx.copy(), ctx_len.copy(), ctx_cap, ver["out_tokens"], ver["out_num"], ver["flags"])
    return dict(draft=draft, draft_len=dlen, feat=feat, alloc=al, verify=ver, ctx=ctx2, ctx_len=len2)
