"""Seeded synthetic workloads for the five step configurations.

Every array is drawn from NumPy's counter-based Philox generator with the seed
``SEED_BASE + 100 * config + stream`` so that a test, the benchmark and the
oracle all see the same bytes.  Nothing here computes any part of the
speculative-decoding step itself: contexts, logits, drafter outputs, uniforms
and tree weights are the step's *inputs*.

Stand-ins (the pages measure on code-editing and chat datasets and trained
models, none of which is used here):

* a copy-heavy context (a random "source" span followed by a copy of it with
  10% of positions replaced) stands in for code-editing requests whose output
  repeats the input;
* a Zipf(1.1) token stream stands in for general text;
* target rows are N(0, 2^2) noise with a large logit planted on a per-request
  "truth" continuation, standing in for a target model that continues the
  text; drafters agree with the truth part of the time.

Logits in bf16 are returned as ``uint16`` bit patterns (round-to-nearest-even
from fp32); ``as_torch_bf16`` turns them into a ``torch.bfloat16`` tensor.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

SEED_BASE = 20261202

# Seed streams.
S_CTX, S_LOGITS, S_DRAFT, S_UNIFORM, S_TREE, S_TRUTH, S_SCORES = 0, 1, 2, 3, 4, 5, 6

# Planted logit for the truth token of a target row: far above the maximum of
# N(0, 2^2) over 151,936 draws (about 8.6), so at T=1 the truth token carries
# roughly 0.9 of the mass.
PLANT_LOGIT = 16.0


def rng_for(config: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(SEED_BASE + 100 * config + stream))


# ---------------------------------------------------------------------------
# estimator coefficients (inputs to the step, stored as fp32)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Estimator:
    """Coefficients theta of the n-gram acceptance estimator.

    Field meaning follows Hybrid Spark, Section 4.2, Eq. (1): one intercept per
    draft position, match-length weights (first / later tokens), agreement
    weight, full-match bonus and copy-length weights (first / later tokens),
    and the reference constants of the features.
    """
    beta: np.ndarray            # [15] float32
    w_first: float = 0.0
    w_rest: float = 0.0
    delta: float = 0.0
    l_first: float = 0.0
    l_rest: float = 0.0
    k_first: float = 0.0
    k_rest: float = 0.0
    n_ref: float = 5.0
    n_full: float = 15.0
    m_ref: float = 15.0
    m_cap: float = 256.0

    def f32(self) -> "Estimator":
        kw = {f.name: np.float32(getattr(self, f.name)) for f in dataclasses.fields(self) if f.name != "beta"}
        return Estimator(beta=np.asarray(self.beta, dtype=np.float32), **kw)


def estimator_qwen3_4b() -> Estimator:
    """Fitted coefficients for Qwen3-4B (Hybrid Spark, Appendix D, Table 5)."""
    beta = [-0.220, 0.155, 0.506, 0.683, 0.788, 0.697, 0.766, 0.721,
            0.631, 0.658, 0.761, 0.803, 0.762, 0.862, 0.811]
    return Estimator(beta=np.array(beta, np.float32), w_first=-0.0893, w_rest=-0.0001,
                     delta=1.2455, l_first=1.1998, l_rest=0.1322,
                     k_first=2.0118, k_rest=1.8333).f32()


def estimator_linear_length(a: float = 0.4, b: float = -1.0) -> Estimator:
    """The calibrated acceptance sigmoid(a * n + b) of the batch-allocation
    workload, written as coefficients: every intercept is a * n_ref + b and both
    match-length weights are a; all other terms are zero."""
    beta = np.full(15, a * 5.0 + b, np.float32)
    return Estimator(beta=beta, w_first=a, w_rest=a).f32()


# ---------------------------------------------------------------------------
# small helpers
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rnd) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_torch_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def uniform_tokens(rng, n, V):
    return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def noisy_copy(rng, src, V, p_replace):
    out = src.copy()
    mask = rng.random(len(src)) < p_replace
    out[mask] = uniform_tokens(rng, int(mask.sum()), V)
    return out


def zipf_sampler(V: int, a: float, rng) -> "callable":
    """Token sampler: Zipf(a) over ranks 1..V mapped to ids by a fixed permutation."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    w = ranks ** (-a)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    perm = rng.permutation(V).astype(np.int32)

    def draw(n, r):
        idx = np.searchsorted(cdf, r.random(n), side="right")
        return perm[np.minimum(idx, V - 1)]
    return draw


def plant_spans(rng, x: np.ndarray, n_spans: int, span: int, live_end: bool):
    """Copy ``n_spans`` spans of ``span`` tokens inside ``x`` (in place).

    Picks 2*n_spans non-overlapping intervals in random positions; interval i
    (a source) is copied onto interval n_spans+i, so every source precedes every
    copy.  With ``live_end`` the last copy ends at the last position.  Returns
    the list of (source_start, copy_start).
    """
    T = len(x)
    k = 2 * n_spans
    free = T - k * span
    assert free >= 0
    n_cuts = k - 1 if live_end else k
    cuts = np.sort(rng.integers(0, free + 1, size=n_cuts))
    edges = np.concatenate([[0], cuts, [free]])
    gaps = np.diff(edges)[:k]
    starts = []
    pos = 0
    for g in gaps:
        pos += int(g)
        starts.append(pos)
        pos += span
    if live_end:
        assert starts[-1] + span == T
    pairs = []
    for i in range(n_spans):
        s, d = starts[i], starts[n_spans + i]
        x[d:d + span] = x[s:s + span]
        pairs.append((s, d))
    return pairs


# ---------------------------------------------------------------------------
# contexts
# ---------------------------------------------------------------------------

def copy_heavy(rng, T, V, src_len, n_truth, p_replace=0.10):
    """A uniform source of ``src_len`` tokens followed by the first
    ``T - src_len`` tokens of a noisy copy of it.  The truth continuation is
    the rest of that noisy copy."""
    src = uniform_tokens(rng, src_len, V)
    cp = noisy_copy(rng, src, V, p_replace)
    n_copy = T - src_len
    assert n_copy + n_truth <= src_len
    ctx = np.concatenate([src, cp[:n_copy]])
    return ctx, cp[n_copy:n_copy + n_truth].copy()


def _contexts(config, BS, T, V, kind, cap=None, n_truth=32, **kw):
    """Build [BS, cap] int32 contexts (zero padded) + lengths + truth continuations."""
    cap = T if cap is None else cap
    rng = rng_for(config, S_CTX)
    trng = rng_for(config, S_TRUTH)
    ctx = np.zeros((BS, cap), np.int32)
    ctx_len = np.full(BS, T, np.int32)
    truth = np.zeros((BS, n_truth), np.int32)
    zipf = None
    if kind == "zipf":
        zipf = zipf_sampler(V, kw.get("zipf_a", 1.1), rng)
    for r in range(BS):
        if kind == "planted":
            x = uniform_tokens(rng, T, V)
            plant_spans(rng, x, kw["n_spans"], kw["span"], live_end=(r % 2 == 0))
            tr = uniform_tokens(trng, n_truth, V)
        elif kind == "copy":
            x, tr = copy_heavy(rng, T, V, kw["src_len"], n_truth)
        elif kind == "half_copy":
            if r % 2 == 0:
                x, tr = copy_heavy(rng, T, V, kw["src_len"], n_truth)
            else:
                x = uniform_tokens(rng, T, V)
                tr = uniform_tokens(trng, n_truth, V)
        elif kind == "zipf":
            x = zipf(T, rng)
            pairs = plant_spans(rng, x, kw["n_spans"], kw["span"], live_end=(r % 2 == 0))
            if r % 2 == 0:
                # the text keeps copying the source of the last planted span
                s, _ = pairs[-1]
                follow = x[s + kw["span"]: s + kw["span"] + n_truth].copy()
                follow = noisy_copy(trng, follow, V, 0.10)
                tr = np.concatenate([follow, zipf(n_truth - len(follow), trng)]) if len(follow) < n_truth else follow
            else:
                tr = zipf(n_truth, trng)
        else:
            raise ValueError(kind)
        ctx[r, :T] = x
        truth[r] = tr
    return ctx, ctx_len, truth


# ---------------------------------------------------------------------------
# logits
# ---------------------------------------------------------------------------

def noise_rows(rng, shape, sigma=2.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def planted_target_rows(rng, truth, n_rows, V, dtype="f32", plant=PLANT_LOGIT):
    """[BS, n_rows, V] target rows: N(0, 2^2) noise, row k planted on truth[k]."""
    BS = truth.shape[0]
    out = np.empty((BS, n_rows, V), np.float32 if dtype == "f32" else np.uint16)
    for r in range(BS):
        z = noise_rows(rng, (n_rows, V))
        z[np.arange(n_rows), truth[r, :n_rows]] = np.float32(plant)
        out[r] = z if dtype == "f32" else f32_to_bf16_bits(z)
    return out


def gumbel_argmax_tokens(rng, w, T):
    """Tokens drawn from softmax(w / T) of each draft row by the Gumbel-max
    trick (the stand-in drafter's own sampling; w: [..., V] float32)."""
    g = -np.log(-np.log(rng.random(w.shape, dtype=np.float64).clip(1e-300, None)))
    return np.argmax(w.astype(np.float64) / T + g, axis=-1).astype(np.int32)


def model_chain_from_truth(rng, truth, K, V, p_agree=0.8):
    d = uniform_tokens(rng, truth.shape[0] * K, V).reshape(truth.shape[0], K)
    agree = rng.random((truth.shape[0], K)) < p_agree
    d[agree] = truth[:, :K][agree]
    return d


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------

def config0(BS=4, V=32000, B=7, T_ctx=512, temperature=1.0):
    """Chain verify, tiny: probabilistic drafts from q, uniforms, planted-span contexts."""
    c = 0
    lrng = rng_for(c, S_LOGITS)
    z = noise_rows(lrng, (BS, B + 1, V))
    w = z[:, :B] + noise_rows(lrng, (BS, B, V), sigma=0.5)
    y = gumbel_argmax_tokens(rng_for(c, S_DRAFT), w, temperature)
    urng = rng_for(c, S_UNIFORM)
    u_acc = urng.random((BS, B), dtype=np.float32)
    u_smp = urng.random(BS, dtype=np.float32)
    ctx, ctx_len, _ = _contexts(c, BS, T_ctx, V, "planted", n_spans=3, span=40)
    return dict(config=c, BS=BS, V=V, B=B, temperature=temperature,
                target=z, draft=w, tokens=y, u_acc=u_acc, u_smp=u_smp,
                ctx=ctx, ctx_len=ctx_len, n_min=3, n_max=3, max_draft=15, copy_cap=256)


def config1(BS=4, V=151936, B=7, T_ctx=4096, src_len=3000, temperature=1.0):
    """Copy-heavy edit workload: model chain as config 0 at full V; the n-gram
    chain (n in {2,3,4}) is verified as point masses against its own rows."""
    c = 1
    lrng = rng_for(c, S_LOGITS)
    z = noise_rows(lrng, (BS, B + 1, V))
    w = z[:, :B] + noise_rows(lrng, (BS, B, V), sigma=0.5)
    y = gumbel_argmax_tokens(rng_for(c, S_DRAFT), w, 1.0)
    ctx, ctx_len, truth = _contexts(c, BS, T_ctx, V, "copy", src_len=src_len)
    ng_rows = planted_target_rows(lrng, truth, 16, V)
    urng = rng_for(c, S_UNIFORM)
    u_acc = urng.random((BS, B), dtype=np.float32)
    u_smp = urng.random(BS, dtype=np.float32)
    u_acc_ng = urng.random((BS, 15), dtype=np.float32)
    u_smp_ng = urng.random(BS, dtype=np.float32)
    return dict(config=c, BS=BS, V=V, B=B, temperature=temperature,
                target=z, draft=w, tokens=y, u_acc=u_acc, u_smp=u_smp,
                ngram_target=ng_rows, u_acc_ng=u_acc_ng, u_smp_ng=u_smp_ng,
                ctx=ctx, ctx_len=ctx_len, truth=truth, ngram_sizes=(2, 3, 4),
                max_draft=15, copy_cap=256)


def config2(BS=128, V=151936, K=7, T_ctx=8192, src_len=6000, budget=256, lam=0.309,
            temperature=1.0, ctx_extra=0):
    """Batch budget allocation at BS 128: bf16 target rows planted on the truth,
    greedy model chain with confidence logits ~N(1,1), n-gram estimator
    sigmoid(0.4 n - 1), global budget of verified draft slots."""
    c = 2
    ctx, ctx_len, truth = _contexts(c, BS, T_ctx, V, "half_copy", cap=T_ctx + ctx_extra, src_len=src_len)
    drng = rng_for(c, S_DRAFT)
    d = model_chain_from_truth(drng, truth, K, V)
    conf = (drng.standard_normal((BS, K), dtype=np.float32) + np.float32(1.0)).astype(np.float32)
    rows = planted_target_rows(rng_for(c, S_LOGITS), truth, 16, V, dtype="bf16")
    urng = rng_for(c, S_UNIFORM)
    return dict(config=c, BS=BS, V=V, K=K, L=15, temperature=temperature, budget=budget, lam=lam,
                ctx=ctx, ctx_len=ctx_len, truth=truth, model_tokens=d, model_conf_logit=conf,
                model_point_mass=np.ones(BS, np.uint8), target_bf16=rows, target_rows_per_req=16,
                u_acc=urng.random((BS, 16), dtype=np.float32), u_smp=urng.random(BS, dtype=np.float32),
                n_min=5, n_max=15, max_draft=15, copy_cap=256, estimator=estimator_linear_length())


def config3_inputs(BS=64, V=151936, P=8, Kc=4, T_ctx=4096, src_len=3000, rows_cap=16,
                   depth_max=32, L=15):
    """Tree verification: drafter block of P positions x Kc ranked candidates,
    n-gram continuations from the anchor and each pick, Exp(1) weights that give
    Dirichlet(1) acceptance estimates over each parent's children plus 'none'.
    Target rows depend on the tree and come from ``tree_target_rows``."""
    c = 3
    ctx, ctx_len, truth = _contexts(c, BS, T_ctx, V, "half_copy", src_len=src_len)
    drng = rng_for(c, S_DRAFT)
    block = np.zeros((BS, P, Kc), np.int32)
    for r in range(BS):
        for i in range(P):
            cand = []
            pick = int(truth[r, i]) if drng.random() < 0.6 else int(drng.integers(0, V))
            cand.append(pick)
            want_truth = pick != truth[r, i] and drng.random() < 0.5
            while len(cand) < Kc:
                t = int(truth[r, i]) if want_truth else int(drng.integers(0, V))
                want_truth = False
                if t not in cand:
                    cand.append(t)
            block[r, i] = cand
    c_max = 1 + P * Kc + (P + 1) * L
    trng = rng_for(c, S_TREE)
    w_node = trng.standard_exponential((BS, c_max), dtype=np.float32)
    w_none = trng.standard_exponential((BS, c_max), dtype=np.float32)
    return dict(config=c, BS=BS, V=V, P=P, Kc=Kc, L=L, rows_cap=rows_cap, depth_max=depth_max,
                c_max=c_max, ctx=ctx, ctx_len=ctx_len, truth=truth, block=block,
                w_node=w_node, w_none=w_none, n_min=3, n_max=15, max_draft=L, copy_cap=256)


def tree_score_inputs(BS, P, Kc, config=3, prior_only=False):
    """Features and coefficients of the Eq. (6) scores for a tree batch: a
    confidence head h and pick share sigma per position, sibling shares r
    (Dirichlet over the siblings), a context term and intercept per request,
    the n-gram source's precision, and coefficients drawn around the
    empty-store prior (pick ln 2 + logit h, sibling log r, the rest 0).  Inputs
    only; the scores are computed by the step."""
    rng = rng_for(config, S_SCORES)
    h = rng.uniform(0.2, 0.95, (BS, P)).astype(np.float32)
    sigma = rng.uniform(0.3, 0.9, (BS, P)).astype(np.float32)
    r = np.zeros((BS, P, Kc), np.float32)
    if Kc > 1:
        r[:, :, 1:] = rng.dirichlet(np.ones(Kc - 1), (BS, P)).astype(np.float32)
    psi_ctx = rng.normal(0, 0.2, BS).astype(np.float32)
    b_req = rng.normal(0, 0.2, BS).astype(np.float32)
    p_src = rng.uniform(0.3, 0.9, BS).astype(np.float32)
    a = np.array([np.log(2.0), 1.0, 0.0, 0.0, 1.0, 0.0, 0.0])
    coef = dict(a=a, w_bucket=np.zeros(64), w_agreed=np.zeros((64, 2)), w_contra=np.zeros((8, 2)),
                psi_depth=np.zeros(16))
    if not prior_only:
        coef = dict(a=a + rng.normal(0, 0.3, 7), w_bucket=rng.normal(0, 0.3, 32),
                    w_agreed=rng.normal(0, 0.3, (32, 2)), w_contra=rng.normal(0, 0.3, (8, 2)),
                    psi_depth=rng.normal(0, 0.1, 16))
        # buckets 32..63: tokens of the follower fallback (drawn last, so the
        # copy buckets keep their values)
        coef["w_bucket"] = np.concatenate([coef["w_bucket"], rng.normal(0, 0.3, 32)])
        coef["w_agreed"] = np.concatenate([coef["w_agreed"], rng.normal(0, 0.3, (32, 2))])
    return dict(coef=coef, h=h, sigma=sigma, r_share=r, psi_ctx=psi_ctx, b_req=b_req, p_src=p_src)


def tree_queries(ctx, ctx_len, block):
    """Query texts for the tree's n-gram chains: query 9r+i (i=0..P) is the
    context of request r followed by the first i picks of its block."""
    BS, P, _ = block.shape
    nq = BS * (P + 1)
    query_req = np.repeat(np.arange(BS, dtype=np.int32), P + 1)
    extra = np.zeros((nq, P), np.int32)
    extra_len = np.zeros(nq, np.int32)
    for r in range(BS):
        for i in range(P + 1):
            q = r * (P + 1) + i
            extra[q, :i] = block[r, :i, 0]
            extra_len[q] = i
    return query_req, extra, extra_len


def tree_target_rows(config, node_token, parent_row, n_rows, truth, V, rows_cap, plant=PLANT_LOGIT):
    """Stand-in target forward over a tree: row i's argmax is the truth token at
    its depth when the path to row i spells the truth, else a random token."""
    BS = node_token.shape[0]
    rng = rng_for(config, S_LOGITS)
    out = np.empty((BS, rows_cap, V), np.float32)
    for r in range(BS):
        z = noise_rows(rng, (rows_cap, V))
        for i in range(int(n_rows[r])):
            path = []
            u = i
            while u > 0:
                path.append(int(node_token[r, u]))
                u = int(parent_row[r, u])
            path.reverse()
            d = len(path)
            on_truth = d < truth.shape[1] and all(path[k] == truth[r, k] for k in range(d))
            tok = int(truth[r, d]) if on_truth else int(rng.integers(0, V))
            z[i, tok] = np.float32(plant)
        out[r] = z
    return out


def config4(BS=256, V=151936, K=7, T_ctx=32768, budget=512, lam=0.309, temperature=0.7, ctx_extra=0):
    """Large-batch stress: Zipf(1.1) contexts with 16 planted 256-token spans,
    bf16 planted target rows, greedy model chain, full Table-5 estimator."""
    c = 4
    ctx, ctx_len, truth = _contexts(c, BS, T_ctx, V, "zipf", cap=T_ctx + ctx_extra, n_spans=16, span=256)
    drng = rng_for(c, S_DRAFT)
    d = model_chain_from_truth(drng, truth, K, V)
    conf = (drng.standard_normal((BS, K), dtype=np.float32) + np.float32(1.0)).astype(np.float32)
    rows = planted_target_rows(rng_for(c, S_LOGITS), truth, 16, V, dtype="bf16")
    urng = rng_for(c, S_UNIFORM)
    return dict(config=c, BS=BS, V=V, K=K, L=15, temperature=temperature, budget=budget, lam=lam,
                ctx=ctx, ctx_len=ctx_len, truth=truth, model_tokens=d, model_conf_logit=conf,
                model_point_mass=np.ones(BS, np.uint8), target_bf16=rows, target_rows_per_req=16,
                u_acc=urng.random((BS, 16), dtype=np.float32), u_smp=urng.random(BS, dtype=np.float32),
                n_min=5, n_max=15, max_draft=15, copy_cap=256, estimator=estimator_qwen3_4b())


def dense_headline(BS=128, V=151936, B=7, T_ctx=8192, src_len=6000, temperature=1.0, ctx_extra=0,
                   config=2):
    """Dense verify + draft at BS 128: bf16 target [BS, B+1, V], draft
    [BS, B, V] = target + N(0, 0.5^2), probabilistic drafts sampled from q,
    then an n-gram draft over the batch-allocation contexts."""
    lrng = rng_for(10 + config, S_LOGITS)
    tgt = np.empty((BS, B + 1, V), np.uint16)
    dft = np.empty((BS, B, V), np.uint16)
    toks = np.empty((BS, B), np.int32)
    drng = rng_for(10 + config, S_DRAFT)
    for r in range(BS):
        z = noise_rows(lrng, (B + 1, V))
        w = z[:B] + noise_rows(lrng, (B, V), sigma=0.5)
        zb = f32_to_bf16_bits(z)
        wb = f32_to_bf16_bits(w)
        tgt[r], dft[r] = zb, wb
        toks[r] = gumbel_argmax_tokens(drng, bf16_bits_to_f32(wb), temperature)
    ctx, ctx_len, _ = _contexts(config, BS, T_ctx, V, "half_copy", cap=T_ctx + ctx_extra, src_len=src_len)
    urng = rng_for(10 + config, S_UNIFORM)
    return dict(BS=BS, V=V, B=B, temperature=temperature, target_bf16=tgt, draft_bf16=dft, tokens=toks,
                u_acc=urng.random((BS, B), dtype=np.float32), u_smp=urng.random(BS, dtype=np.float32),
                ctx=ctx, ctx_len=ctx_len, n_min=5, n_max=15, max_draft=15, copy_cap=256)


# ---------------------------------------------------------------------------
# a batch served over several steps (the host's sizing loop)
# ---------------------------------------------------------------------------

class ServingLoop:
    """Requests served over several steps.  Each request's output follows a
    fixed stream: for the first half, the rest of a passage that its prompt
    holds once in full and ends by repeating the passage's opening (so the
    n-gram drafter can continue it), for the rest random tokens.  A step's
    inputs are its raw draws (``step_raw``) put in place by how many tokens
    each request has emitted so far (``assemble``): a greedy model chain that
    agrees with the stream at rate p_agree, its confidence logits ~ N(1, 1),
    and fp32 target rows of N(0, 2^2) noise whose row k is planted on the
    stream's token k from the current position (argmax at T = 0)."""

    def __init__(self, BS=32, V=1024, T_prompt=600, passage=240, steps=8, K=7, rows=16, config=7, p_agree=0.8):
        self.BS, self.V, self.K, self.rows, self.steps = BS, V, K, rows, steps
        self.T_prompt, self.config, self.p_agree = T_prompt, config, p_agree
        rng = rng_for(config, S_CTX)
        self.cap = T_prompt + steps * rows
        self.ctx = np.zeros((BS, self.cap), np.int32)
        self.ctx_len = np.full(BS, T_prompt, np.int32)
        span = steps * rows + rows
        self.stream = np.zeros((BS, span), np.int32)
        for r in range(BS):
            if r < BS // 2:
                p = uniform_tokens(rng, passage, V)
                head = int(rng.integers(20, 60))
                pre = uniform_tokens(rng, T_prompt - passage - head - 40, V)
                mid = uniform_tokens(rng, 40, V)
                self.ctx[r, :T_prompt] = np.concatenate([pre, p, mid, p[:head]])
                tail = p[head:]
                self.stream[r] = np.concatenate([tail, uniform_tokens(rng, max(0, span - len(tail)), V)])[:span]
            else:
                self.ctx[r, :T_prompt] = uniform_tokens(rng, T_prompt, V)
                self.stream[r] = uniform_tokens(rng, span, V)

    def step_raw(self, t):
        BS, K, V = self.BS, self.K, self.V
        drng = rng_for(self.config, 100 + 3 * t + S_DRAFT)
        rand = uniform_tokens(drng, BS * K, V).reshape(BS, K)
        agree = drng.random((BS, K)) < self.p_agree
        conf = (drng.standard_normal((BS, K), dtype=np.float32) + np.float32(1.0)).astype(np.float32)
        noise = noise_rows(rng_for(self.config, 100 + 3 * t + S_LOGITS), (BS, self.rows, V))
        return dict(rand=rand, agree=agree, conf=conf, noise=noise)

    def assemble(self, raw, emitted):
        """The step's inputs given the tokens each request has emitted."""
        BS, K, rows = self.BS, self.K, self.rows
        truth = np.stack([self.stream[r, emitted[r]:emitted[r] + rows] for r in range(BS)])
        model = np.where(raw["agree"], truth[:, :K], raw["rand"]).astype(np.int32)
        target = raw["noise"].copy()
        for r in range(BS):
            target[r, np.arange(rows), truth[r]] = np.float32(PLANT_LOGIT)
        return dict(model_tokens=model, model_conf_logit=raw["conf"], target=target.reshape(BS * rows, self.V))
