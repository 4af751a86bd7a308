"""ctypes binding of ``libspec_hip.so`` (the C ABI declared in include/spec.h).

Argument marshalling only: every function takes ``torch`` device tensors,
allocates outputs and workspace with torch (device memory plumbing), and calls
the C entry point of the same name on the current HIP stream.  No step of the
method runs here, and there is no fallback: if the library is missing the
import fails.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec_hip.so")

i32, i64, f32, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t

# ---- constants mirrored from spec.h ----------------------------------------
SPEC_OK, SPEC_EINVAL, SPEC_EWORKSPACE, SPEC_EHIP = 0, -1, -2, -3
SPEC_F32, SPEC_BF16 = 0, 1
FLAG_RESIDUAL_ZERO, FLAG_BAD_TOKEN, FLAG_BAD_LOGITS, FLAG_CTX_OVERFLOW, FLAG_BAD_LENGTH, FLAG_RESIDUAL_LATE = (
    1 << 5, 1 << 8, 1 << 9, 1 << 10, 1 << 11, 1 << 12)
SLOT_POINT_MASS, SLOT_FROM_NGRAM = 1, 2
SRC_MODEL, SRC_NGRAM, SRC_MERGED, SRC_EXTENDED = 0, 1, 2, 3
POLICIES = {"proposed": 0, "ngram_first": 1, "extension": 2, "model_only": 3, "ngram_only": 4}
ALLOC_CHAIN, ALLOC_TREE = 0, 1
OP_NGRAM, OP_ALLOCATE, OP_VERIFY_CHAIN, OP_VERIFY_TREE = 0, 1, 2, 3
MAX_DRAFT, MAX_CAP, MAX_ROWS, MAX_FOREST, MAX_VOCAB = 32, 1024, 64, 1024, 8388608


class NgramArgs(C.Structure):
    _fields_ = [("bs", i32), ("nq", i32), ("ctx", vp), ("ctx_stride", i64), ("ctx_len", vp),
                ("query_req", vp), ("extra", vp), ("extra_stride", i64), ("extra_len", vp),
                ("n_min", i32), ("n_max", i32), ("max_draft", i32), ("copy_cap", i32), ("follow_ctx", i32),
                ("draft", vp), ("draft_len", vp), ("feat", vp), ("draft_follow", vp), ("workspace", vp),
                ("workspace_bytes", sz)]


class Estimator(C.Structure):
    _fields_ = [("beta", f32 * 15)] + [(n, f32) for n in (
        "w_first", "w_rest", "delta", "l_first", "l_rest", "k_first", "k_rest",
        "n_ref", "n_full", "m_ref", "m_cap")]


class ChainAlloc(C.Structure):
    _fields_ = [("bs", i32), ("K", i32), ("ld", i32), ("model_tokens", vp), ("model_conf", vp),
                ("conf_is_logit", i32), ("model_point_mass", vp), ("ngram_draft", vp), ("ngram_ld", i32),
                ("ngram_len", vp), ("ngram_feat", vp), ("est", Estimator), ("lam", f32), ("budget", i32),
                ("policy", i32), ("chain_tokens", vp), ("slot_flags", vp), ("chain_len", vp), ("chain_src", vp),
                ("survival", vp), ("alloc_len", vp), ("row_base", vp), ("total_rows", vp), ("out_flags", vp)]


class TreeScores(C.Structure):
    _fields_ = [("a", C.c_double * 7), ("w_bucket", C.c_double * 64), ("w_agreed", (C.c_double * 2) * 64),
                ("w_contra", (C.c_double * 2) * 8), ("psi_depth", C.c_double * 16), ("h", vp), ("sigma", vp),
                ("r_share", vp), ("psi_ctx", vp), ("b_req", vp), ("p_src", vp), ("ngram_feat", vp)]


class TreeAlloc(C.Structure):
    _fields_ = [("bs", i32), ("P", i32), ("Kc", i32), ("block", vp), ("ngram_draft", vp), ("ngram_ld", i32),
                ("ngram_len", vp), ("ngram_follow", vp), ("w_node", vp), ("w_none", vp), ("scores", vp),
                ("c_max", i32),
                ("depth_max", i32), ("rows_cap", i32), ("node_token", vp), ("parent_row", vp), ("Q", vp),
                ("n_rows", vp), ("row_base", vp), ("total_rows", vp), ("forest_count", vp), ("s_curve", vp),
                ("out_flags", vp), ("forest_token", vp), ("forest_parent", vp), ("forest_q", vp), ("forest_n", vp)]


class AllocArgs(C.Structure):
    _fields_ = [("mode", i32), ("chain", ChainAlloc), ("tree", TreeAlloc), ("workspace", vp),
                ("workspace_bytes", sz)]


class VerifyArgs(C.Structure):
    _fields_ = [("bs", i32), ("vocab", i32), ("temperature", f32), ("logits", vp), ("dtype", i32),
                ("row_stride", i64), ("row_base", vp), ("n_logit_rows", i64), ("draft_logits", vp),
                ("draft_dtype", i32), ("draft_row_stride", i64), ("draft_row_base", vp), ("n_draft_rows", i64),
                ("tokens", vp), ("slot_flags", vp), ("ld", i32), ("n_slots", vp), ("max_slots", i32), ("u_accept", vp),
                ("u_sample", vp), ("rng", i32), ("rng_seed", C.c_uint64), ("rng_offset", C.c_uint64),
                ("out_tokens", vp), ("out_num", vp), ("out_accepted", vp), ("out_p", vp),
                ("out_q", vp), ("out_flags", vp), ("write_flags", i32), ("out_accept_hist", vp), ("ctx", vp),
                ("ctx_stride", i64),
                ("ctx_len", vp), ("ctx_len_out", vp), ("ctx_cap", i32), ("ngram_draft", vp),
                ("ngram_draft_len", vp), ("ngram_feat", vp), ("ngram_n_min", i32), ("ngram_n_max", i32),
                ("ngram_max_draft", i32), ("ngram_copy_cap", i32), ("residual_wait", i32), ("prof_begin", vp),
                ("prof_end", vp),
                ("workspace", vp), ("workspace_bytes", sz)]


class TreeVerifyArgs(C.Structure):
    _fields_ = [("bs", i32), ("vocab", i32), ("rows_max", i32), ("logits", vp), ("dtype", i32),
                ("row_stride", i64), ("row_base", vp), ("n_logit_rows", i64), ("node_token", vp),
                ("parent_row", vp), ("n_rows", vp), ("out_tokens", vp), ("out_num", vp), ("out_path_rows", vp),
                ("out_argmax", vp), ("out_flags", vp), ("ctx", vp), ("ctx_stride", i64), ("ctx_len", vp),
                ("ctx_len_out", vp), ("ctx_cap", i32), ("prof_begin", vp), ("prof_end", vp), ("workspace", vp),
                ("workspace_bytes", sz)]


class CostModel(C.Structure):
    _fields_ = [("c0", C.c_double), ("p", C.c_double), ("graph_limit", i32), ("n_tokens", i32), ("eager", vp),
                ("n_eager", i32)]


STRUCTS = {"spec_cost_model": CostModel, "spec_tree_scores": TreeScores, "spec_ngram_args": NgramArgs, "spec_estimator": Estimator, "spec_chain_alloc": ChainAlloc,
           "spec_tree_alloc": TreeAlloc, "spec_alloc_args": AllocArgs, "spec_verify_args": VerifyArgs,
           "spec_tree_verify_args": TreeVerifyArgs}
EXPORTS = ("spec_size_budget", "spec_ngram_draft", "spec_allocate_budget", "spec_verify_chain", "spec_verify_tree",
           "spec_verify_chain_noalloc", "spec_workspace_bytes", "spec_strerror", "spec_last_hip_error",
           "spec_abi_version")
NOALLOC_SCRATCH_BYTES = 16 << 20


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                          "(the HIP path has no fallback)")
    lib = C.CDLL(path)
    for name in ("spec_ngram_draft", "spec_allocate_budget", "spec_verify_chain", "spec_verify_tree",
                 "spec_verify_chain_noalloc"):
        getattr(lib, name).argtypes = [vp, vp]
        getattr(lib, name).restype = C.c_int
    lib.spec_workspace_bytes.argtypes = [C.c_int, vp]
    lib.spec_workspace_bytes.restype = sz
    lib.spec_strerror.argtypes = [C.c_int]
    lib.spec_strerror.restype = C.c_char_p
    lib.spec_last_hip_error.restype = C.c_char_p
    lib.spec_abi_version.restype = C.c_int
    lib.spec_size_budget.argtypes = [vp, C.c_int64, C.c_int32, vp, C.c_int32, vp, vp, vp, vp]
    lib.spec_size_budget.restype = C.c_int
    return lib


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims")
    return t


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def _check(rc: int):
    if rc != SPEC_OK:
        l = lib()
        msg = l.spec_strerror(rc).decode()
        if rc == SPEC_EHIP:
            msg += ": " + l.spec_last_hip_error().decode()
        raise RuntimeError(f"libspec_hip: {msg} (code {rc})")


def _workspace(op, args, device, workspace, stream=None):
    """The call's workspace: the caller's, or a new one from torch's caching
    allocator.  A new one is dropped when the call returns, so when the call
    runs on another stream than the current one the block is recorded on that
    stream (the allocator then does not hand it out again until the stream's
    work is done)."""
    need = lib().spec_workspace_bytes(op, C.byref(args))
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=device)
        if stream is not None:
            workspace.record_stream(stream)
    elif workspace.numel() < need + 256:
        raise ValueError(f"workspace too small: {workspace.numel()} < {need + 256}")
    base = workspace.data_ptr()
    aligned = (base + 255) // 256 * 256
    return workspace, (aligned, need)


def _logits_dtype(t):
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _rows2d(t, name):
    if t.dim() < 2:
        raise ValueError(f"{name} must be [..., V]")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    t2 = t.reshape(-1, t.shape[-1]) if t.is_contiguous() else t
    if t2.dim() != 2:
        raise ValueError(f"{name} must be reshapeable to [rows, V]")
    return t2


def estimator_struct(est) -> Estimator:
    s = Estimator()
    for i in range(15):
        s.beta[i] = float(est.beta[i])
    for n in ("w_first", "w_rest", "delta", "l_first", "l_rest", "k_first", "k_rest",
              "n_ref", "n_full", "m_ref", "m_cap"):
        setattr(s, n, float(getattr(est, n)))
    return s


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def spec_size_budget(survival, n_requests, c0, p, b_max=0, graph_limit=0, n_tokens=0, eager=None, curve=False):
    """Budget sizing on the host from a host copy of the survivals: returns
    (b*, lambda, G(b*)) and, with ``curve``, G(b) for every b as well."""
    import numpy as np
    s = np.ascontiguousarray(np.ravel(survival.cpu().numpy() if isinstance(survival, torch.Tensor) else survival),
                             dtype=np.float32)
    eg = None if eager is None else np.ascontiguousarray(eager, dtype=np.float64)
    cm = CostModel(float(c0), float(p), int(graph_limit), int(n_tokens),
                   None if eg is None else eg.ctypes.data_as(vp), 0 if eg is None else len(eg))
    top = len(s) if b_max <= 0 or b_max > len(s) else int(b_max)
    g = np.empty(top + 1, np.float64) if curve else None
    b, lam, gb = C.c_int32(0), C.c_double(0.0), C.c_double(0.0)
    _check(lib().spec_size_budget(s.ctypes.data_as(vp), len(s), int(n_requests), C.byref(cm), int(b_max),
                                  C.byref(b), C.byref(lam), C.byref(gb), None if g is None else g.ctypes.data_as(vp)))
    return (b.value, lam.value, gb.value, g) if curve else (b.value, lam.value, gb.value)


def spec_ngram_draft(ctx, ctx_len, n_min, n_max, max_draft=15, copy_cap=256, query_req=None, extra=None,
                     extra_len=None, out=None, workspace=None, stream=None, follow_ctx=0):
    """N-gram drafts for every query; returns (draft [nq, max_draft], draft_len [nq], feat [nq, 4]), and with
    follow_ctx > 0 (the follower fallback) also the follower counts [nq, max_draft]."""
    _dev(ctx, torch.int32, "ctx", 2)
    _dev(ctx_len, torch.int32, "ctx_len", 1)
    dev = ctx.device
    nq = query_req.shape[0] if query_req is not None else ctx.shape[0]
    if query_req is not None:
        _dev(query_req, torch.int32, "query_req", 1)
    if extra is not None:
        _dev(extra, torch.int32, "extra", 2)
        _dev(extra_len, torch.int32, "extra_len", 1)
    if out is None:
        out = (torch.empty((nq, max_draft), dtype=torch.int32, device=dev),
               torch.empty(nq, dtype=torch.int32, device=dev),
               torch.empty((nq, 4), dtype=torch.int32, device=dev))
        if follow_ctx > 0:
            out += (torch.empty((nq, max_draft), dtype=torch.int32, device=dev),)
    draft, dlen, feat = out[:3]
    fol = out[3] if len(out) > 3 else None
    a = NgramArgs(bs=ctx.shape[0], nq=nq, ctx=_ptr(ctx), ctx_stride=ctx.shape[1], ctx_len=_ptr(ctx_len),
                  query_req=_ptr(query_req), extra=_ptr(extra),
                  extra_stride=0 if extra is None else extra.shape[1], extra_len=_ptr(extra_len),
                  n_min=n_min, n_max=n_max, max_draft=max_draft, copy_cap=copy_cap, follow_ctx=follow_ctx,
                  draft=_ptr(draft), draft_len=_ptr(dlen), feat=_ptr(feat), draft_follow=_ptr(fol))
    ws, w = _workspace(OP_NGRAM, a, dev, workspace, stream)
    if w:
        a.workspace, a.workspace_bytes = w
    _check(lib().spec_ngram_draft(C.byref(a), _stream(dev, stream)))
    return (draft, dlen, feat, fol) if fol is not None else (draft, dlen, feat)


def _chain_alloc(model_tokens, model_conf, ngram_draft, ngram_len, ngram_feat, est, lam, budget,
                 policy="proposed", conf_is_logit=True, model_point_mass=None, ld=15, out=None,
                 workspace=None, stream=None):
    _dev(model_tokens, torch.int32, "model_tokens", 2)
    _dev(model_conf, torch.float32, "model_conf", 2)
    _dev(ngram_draft, torch.int32, "ngram_draft", 2)
    _dev(ngram_len, torch.int32, "ngram_len", 1)
    _dev(ngram_feat, torch.int32, "ngram_feat", 2)
    if model_point_mass is not None:
        _dev(model_point_mass, torch.uint8, "model_point_mass", 1)
    bs, K = model_tokens.shape
    dev = model_tokens.device
    if out is None:
        out = dict(chain_tokens=torch.empty((bs, ld), dtype=torch.int32, device=dev),
                   slot_flags=torch.empty((bs, ld), dtype=torch.uint8, device=dev),
                   chain_len=torch.empty(bs, dtype=torch.int32, device=dev),
                   chain_src=torch.empty(bs, dtype=torch.int32, device=dev),
                   survival=torch.empty((bs, ld), dtype=torch.float32, device=dev),
                   alloc_len=torch.empty(bs, dtype=torch.int32, device=dev),
                   row_base=torch.empty(bs, dtype=torch.int64, device=dev),
                   total_rows=torch.empty(1, dtype=torch.int32, device=dev),
                   out_flags=torch.empty(bs, dtype=torch.int32, device=dev))
    ca = ChainAlloc(bs=bs, K=K, ld=ld, model_tokens=_ptr(model_tokens), model_conf=_ptr(model_conf),
                    conf_is_logit=int(conf_is_logit), model_point_mass=_ptr(model_point_mass),
                    ngram_draft=_ptr(ngram_draft), ngram_ld=ngram_draft.shape[1], ngram_len=_ptr(ngram_len),
                    ngram_feat=_ptr(ngram_feat), est=estimator_struct(est), lam=float(lam), budget=int(budget),
                    policy=POLICIES[policy] if isinstance(policy, str) else int(policy),
                    **{k: _ptr(v) for k, v in out.items()})
    a = AllocArgs(mode=ALLOC_CHAIN, chain=ca)
    ws, w = _workspace(OP_ALLOCATE, a, dev, workspace, stream)
    if w:
        a.workspace, a.workspace_bytes = w
    _check(lib().spec_allocate_budget(C.byref(a), _stream(dev, stream)))
    return out


def tree_scores_struct(coef, h, sigma, r_share, psi_ctx, b_req, p_src, ngram_feat):
    """spec_tree_scores: coefficient tables from ``coef`` (a [7], w_bucket [64],
    w_agreed [64, 2], w_contra [8, 2], psi_depth [16]) and device feature tensors."""
    for t, name in ((h, "h"), (sigma, "sigma"), (r_share, "r_share"), (psi_ctx, "psi_ctx"), (b_req, "b_req"),
                    (p_src, "p_src")):
        _dev(t, torch.float32, name)
    _dev(ngram_feat, torch.int32, "ngram_feat", 2)
    st = TreeScores()
    st.a[:] = [float(x) for x in coef["a"]]
    st.w_bucket[:] = [float(x) for x in coef["w_bucket"]]
    for i in range(64):
        st.w_agreed[i][:] = [float(x) for x in coef["w_agreed"][i]]
    for i in range(8):
        st.w_contra[i][:] = [float(x) for x in coef["w_contra"][i]]
    st.psi_depth[:] = [float(x) for x in coef["psi_depth"]]
    st.h, st.sigma, st.r_share = _ptr(h), _ptr(sigma), _ptr(r_share)
    st.psi_ctx, st.b_req, st.p_src, st.ngram_feat = _ptr(psi_ctx), _ptr(b_req), _ptr(p_src), _ptr(ngram_feat)
    return st


def _tree_alloc(block=None, ngram_draft=None, ngram_len=None, w_node=None, w_none=None, depth_max=32, rows_cap=16,
                out=None, stream=None, scores=None, c_max=None, s_curve=False, ngram_follow=None, forest=None):
    """Tree build; weights w_node / w_none by candidate index, or ``scores``
    (the keyword arguments of tree_scores_struct) for the Eq. (6) form.  With
    ``s_curve`` the S(n) curve [bs, rows_cap] is returned as out["s_curve"].
    ``ngram_follow``: the chains' follower counts (spec_ngram_draft with
    follow_ctx), or None when every chain token is copied.  ``forest``: a
    caller-built forest (token int32 [bs, c_max], parent int32 [bs, c_max],
    q float32 [bs, c_max], n int32 [bs]) instead of block and chains."""
    if forest is not None:
        return _tree_from_forest(forest, rows_cap, out, stream, s_curve)
    _dev(block, torch.int32, "block", 3)
    _dev(ngram_draft, torch.int32, "ngram_draft", 2)
    _dev(ngram_len, torch.int32, "ngram_len", 1)
    if ngram_follow is not None:
        _dev(ngram_follow, torch.int32, "ngram_follow", 2)
        if tuple(ngram_follow.shape) != tuple(ngram_draft.shape):
            raise ValueError("ngram_follow must have ngram_draft's shape")
    if scores is None:
        _dev(w_node, torch.float32, "w_node", 2)
        _dev(w_none, torch.float32, "w_none", 2)
        c_max = w_node.shape[1]
    elif c_max is None:
        raise ValueError("c_max is needed with scores")
    bs, P, Kc = block.shape
    dev = block.device
    if out is None:
        out = _tree_outputs(bs, rows_cap, dev, s_curve)
    st = None if scores is None else tree_scores_struct(**scores)
    ta = TreeAlloc(bs=bs, P=P, Kc=Kc, block=_ptr(block), ngram_draft=_ptr(ngram_draft),
                   ngram_ld=ngram_draft.shape[1], ngram_len=_ptr(ngram_len), ngram_follow=_ptr(ngram_follow),
                   w_node=_ptr(w_node),
                   w_none=_ptr(w_none), scores=None if st is None else C.cast(C.pointer(st), vp),
                   c_max=int(c_max), depth_max=depth_max, rows_cap=rows_cap,
                   **{k: _ptr(v) for k, v in out.items()})
    a = AllocArgs(mode=ALLOC_TREE, tree=ta)
    _check(lib().spec_allocate_budget(C.byref(a), _stream(dev, stream)))
    return out


def _tree_outputs(bs, rows_cap, dev, s_curve):
    out = dict(node_token=torch.empty((bs, rows_cap), dtype=torch.int32, device=dev),
               parent_row=torch.empty((bs, rows_cap), dtype=torch.int32, device=dev),
               Q=torch.empty((bs, rows_cap), dtype=torch.float32, device=dev),
               n_rows=torch.empty(bs, dtype=torch.int32, device=dev),
               row_base=torch.empty(bs, dtype=torch.int64, device=dev),
               total_rows=torch.empty(1, dtype=torch.int32, device=dev),
               forest_count=torch.empty(bs, dtype=torch.int32, device=dev),
               out_flags=torch.empty(bs, dtype=torch.int32, device=dev))
    if s_curve:
        out["s_curve"] = torch.empty((bs, rows_cap), dtype=torch.float32, device=dev)
    return out


def _tree_from_forest(forest, rows_cap, out, stream, s_curve):
    token, parent, q, n = forest
    _dev(token, torch.int32, "forest token", 2)
    _dev(parent, torch.int32, "forest parent", 2)
    _dev(q, torch.float32, "forest q", 2)
    _dev(n, torch.int32, "forest n", 1)
    bs, c_max = token.shape
    if tuple(parent.shape) != (bs, c_max) or tuple(q.shape) != (bs, c_max) or n.shape[0] != bs:
        raise ValueError("forest token, parent and q must be [bs, c_max] and n [bs]")
    if out is None:
        out = _tree_outputs(bs, rows_cap, token.device, s_curve)
    ta = TreeAlloc(bs=bs, c_max=int(c_max), rows_cap=rows_cap, forest_token=_ptr(token), forest_parent=_ptr(parent),
                   forest_q=_ptr(q), forest_n=_ptr(n), **{k: _ptr(v) for k, v in out.items()})
    a = AllocArgs(mode=ALLOC_TREE, tree=ta)
    _check(lib().spec_allocate_budget(C.byref(a), _stream(token.device, stream)))
    return out


def spec_allocate_budget(mode="chain", **kw):
    """Chain mode: chain selection + budget allocation; tree mode: best-first tree build."""
    if mode == "chain":
        return _chain_alloc(**kw)
    if mode == "tree":
        return _tree_alloc(**kw)
    raise ValueError(mode)


def spec_verify_chain(logits, row_base, tokens, n_slots, temperature, u_accept=None, u_sample=None,
                      slot_flags=None, draft_logits=None, draft_row_base=None, out_flags=None,
                      ctx=None, ctx_len=None, ctx_cap=None, ctx_len_out=None, out=None, workspace=None,
                      stream=None, prof_events=None, max_slots=0, write_flags=False, ngram=None, ngram_out=None,
                      rng=None, accept_hist=None, residual_wait=0, noalloc=False):
    """Rejection-sampling verification of one chain per request (optional commit into ctx).
    ``prof_events``: optional pair of raw hipEvent_t handles recorded around the
    row-statistics pass.  ``max_slots``: optional bound of the total slots
    (e.g. the allocation budget), which sizes the statistics grid.
    ``write_flags``: out_flags receive this call's flags instead of OR-ing
    them in (a new out_flags tensor is then not zeroed first).
    ``ngram``: optional (n_min, n_max, max_draft, copy_cap): with a commit, the
    next n-gram draft of every request over its committed context is computed
    in the same launch and returned as out["ngram_draft"], out["ngram_len"],
    out["ngram_feat"] (into ``ngram_out``, a (draft, len, feat) triple, if given).
    ``rng``: optional (seed, offset): the call draws its uniforms with
    Philox4x32-10 instead of reading u_accept / u_sample.  ``accept_hist``:
    optional int32 [ld + 1] device tensor, increased at each request's
    accepted count.  ``residual_wait``: polls of a published residual sum
    before the drawing workgroup sums the residual itself (0 = the library's
    default; negative = at once, which tests the fallback).  ``noalloc``: call
    spec_verify_chain_noalloc, whose scratch is the library's own per-device
    array (no workspace is allocated or passed; pass ``out`` and
    ``out_flags`` for a call that allocates nothing at all)."""
    lg = _rows2d(logits, "logits")
    _dev(row_base, torch.int64, "row_base", 1)
    _dev(tokens, torch.int32, "tokens", 2)
    _dev(n_slots, torch.int32, "n_slots", 1)
    bs, ld = tokens.shape
    dev = tokens.device
    if slot_flags is not None:
        _dev(slot_flags, torch.uint8, "slot_flags", 2)
    if u_accept is not None:
        _dev(u_accept, torch.float32, "u_accept", 2)
        if u_accept.shape != (bs, ld):
            raise ValueError("u_accept must be [bs, ld]")
        _dev(u_sample, torch.float32, "u_sample", 1)
    dl = None
    if draft_logits is not None:
        dl = _rows2d(draft_logits, "draft_logits")
        _dev(draft_row_base, torch.int64, "draft_row_base", 1)
    if out is None:
        out = dict(out_tokens=torch.empty((bs, ld + 1), dtype=torch.int32, device=dev),
                   out_num=torch.empty(bs, dtype=torch.int32, device=dev),
                   out_accepted=torch.empty(bs, dtype=torch.int32, device=dev),
                   out_p=torch.empty((bs, ld + 1), dtype=torch.float32, device=dev),
                   out_q=torch.empty((bs, ld), dtype=torch.float32, device=dev))
    if out_flags is None:
        out_flags = (torch.empty if write_flags else torch.zeros)(bs, dtype=torch.int32, device=dev)
    out["out_flags"] = out_flags
    a = VerifyArgs(bs=bs, vocab=lg.shape[1], temperature=float(temperature), logits=_ptr(lg),
                   dtype=_logits_dtype(lg), row_stride=lg.stride(0), row_base=_ptr(row_base),
                   n_logit_rows=lg.shape[0], tokens=_ptr(tokens), slot_flags=_ptr(slot_flags), ld=ld,
                   n_slots=_ptr(n_slots), max_slots=int(max_slots), u_accept=_ptr(u_accept),
                   u_sample=_ptr(u_sample),
                   write_flags=int(bool(write_flags)), residual_wait=int(residual_wait),
                   **{k: _ptr(v) for k, v in out.items()})
    if dl is not None:
        a.draft_logits, a.draft_dtype, a.draft_row_stride = _ptr(dl), _logits_dtype(dl), dl.stride(0)
        a.draft_row_base, a.n_draft_rows = _ptr(draft_row_base), dl.shape[0]
    if ctx is not None:
        _dev(ctx, torch.int32, "ctx", 2)
        _dev(ctx_len, torch.int32, "ctx_len", 1)
        a.ctx, a.ctx_stride, a.ctx_len = _ptr(ctx), ctx.shape[1], _ptr(ctx_len)
        a.ctx_cap = ctx.shape[1] if ctx_cap is None else int(ctx_cap)
        if ctx_len_out is not None:
            _dev(ctx_len_out, torch.int32, "ctx_len_out", 1)
            a.ctx_len_out = _ptr(ctx_len_out)
    if rng is not None:
        a.rng, a.rng_seed, a.rng_offset = 1, int(rng[0]) & (2**64 - 1), int(rng[1]) & (2**64 - 1)
    if accept_hist is not None:
        _dev(accept_hist, torch.int32, "accept_hist", 1)
        if accept_hist.shape[0] < ld + 1:
            raise ValueError("accept_hist must hold ld + 1 counts")
        a.out_accept_hist = _ptr(accept_hist)
    if ngram is not None:
        if ctx is None:
            raise ValueError("the fused n-gram draft needs the commit (ctx)")
        n_min, n_max, max_draft, copy_cap = (int(x) for x in ngram)
        if ngram_out is None:
            ngram_out = (torch.empty((bs, max_draft), dtype=torch.int32, device=dev),
                         torch.empty(bs, dtype=torch.int32, device=dev),
                         torch.empty((bs, 4), dtype=torch.int32, device=dev))
        nd, nl, nf = ngram_out
        a.ngram_draft, a.ngram_draft_len, a.ngram_feat = _ptr(nd), _ptr(nl), _ptr(nf)
        a.ngram_n_min, a.ngram_n_max, a.ngram_max_draft, a.ngram_copy_cap = n_min, n_max, max_draft, copy_cap
    if prof_events is not None:
        a.prof_begin, a.prof_end = prof_events
    if noalloc:
        _check(lib().spec_verify_chain_noalloc(C.byref(a), _stream(dev, stream)))
    else:
        ws, w = _workspace(OP_VERIFY_CHAIN, a, dev, workspace, stream)
        if w:
            a.workspace, a.workspace_bytes = w
        _check(lib().spec_verify_chain(C.byref(a), _stream(dev, stream)))
    if ngram is not None:
        out["ngram_draft"], out["ngram_len"], out["ngram_feat"] = ngram_out
    return out


def spec_verify_tree(logits, row_base, node_token, parent_row, n_rows, out_flags=None, ctx=None, ctx_len=None,
                     ctx_cap=None, ctx_len_out=None, out=None, workspace=None, stream=None, prof_events=None):
    """Greedy verification of one tree per request (optional commit into ctx)."""
    lg = _rows2d(logits, "logits")
    _dev(row_base, torch.int64, "row_base", 1)
    _dev(node_token, torch.int32, "node_token", 2)
    _dev(parent_row, torch.int32, "parent_row", 2)
    _dev(n_rows, torch.int32, "n_rows", 1)
    bs, rm = node_token.shape
    dev = node_token.device
    if out is None:
        out = dict(out_tokens=torch.empty((bs, rm), dtype=torch.int32, device=dev),
                   out_num=torch.empty(bs, dtype=torch.int32, device=dev),
                   out_path_rows=torch.empty((bs, rm), dtype=torch.int32, device=dev),
                   out_argmax=torch.empty((bs, rm), dtype=torch.int32, device=dev))
    if out_flags is None:
        out_flags = torch.zeros(bs, dtype=torch.int32, device=dev)
    out["out_flags"] = out_flags
    a = TreeVerifyArgs(bs=bs, vocab=lg.shape[1], rows_max=rm, logits=_ptr(lg), dtype=_logits_dtype(lg),
                       row_stride=lg.stride(0), row_base=_ptr(row_base), n_logit_rows=lg.shape[0],
                       node_token=_ptr(node_token), parent_row=_ptr(parent_row), n_rows=_ptr(n_rows),
                       **{k: _ptr(v) for k, v in out.items()})
    if ctx is not None:
        _dev(ctx, torch.int32, "ctx", 2)
        _dev(ctx_len, torch.int32, "ctx_len", 1)
        a.ctx, a.ctx_stride, a.ctx_len = _ptr(ctx), ctx.shape[1], _ptr(ctx_len)
        a.ctx_cap = ctx.shape[1] if ctx_cap is None else int(ctx_cap)
        if ctx_len_out is not None:
            _dev(ctx_len_out, torch.int32, "ctx_len_out", 1)
            a.ctx_len_out = _ptr(ctx_len_out)
    if prof_events is not None:
        a.prof_begin, a.prof_end = prof_events
    ws, w = _workspace(OP_VERIFY_TREE, a, dev, workspace, stream)
    if w:
        a.workspace, a.workspace_bytes = w
    _check(lib().spec_verify_tree(C.byref(a), _stream(dev, stream)))
    return out
