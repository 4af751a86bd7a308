/*
 * spec.h -- C ABI of the GPU-resident speculative-decoding step for MI355X
 * (gfx950): n-gram draft, verification-budget allocation (chains and trees),
 * lossless chain verification by rejection sampling, greedy tree
 * verification.
 *
 * Sources (page titles):
 *   [HS] "Hybrid Spark: Adaptive Speculative Decoding That Lets the Content
 *        Choose the Drafter"
 *   [AS] "AdaSpark: Adaptive DSpark with Online Learning for Tree Verification
 *        and N-gram Fill"
 *   [LS] "Efficient speculative decoding with a fixed-cost parallel drafter"
 *        (LongSpark), Section 2.1
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device (or managed) memory; everything
 *   else is host memory read during the call.  The caller owns every buffer.
 *   The library allocates nothing: scratch memory comes from the caller's
 *   `workspace` (query its size with spec_workspace_bytes; any alignment of
 *   256 bytes is enough), or for spec_verify_chain_noalloc from a fixed array
 *   per device.  Its only state between calls: caches of device properties
 *   that do not change while the process runs (compute units per device,
 *   resident workgroups per kernel, that array's device address), filled
 *   once under a lock.
 * - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *   and the call returns at once.  The library never synchronises, never
 *   copies device to host and never calls hipDeviceSynchronize, so a whole
 *   step can be captured in a HIP graph.
 * - Return value: SPEC_OK, or a negative code.  A host-detectable error
 *   (null pointer, bad size, bad enum, short workspace) enqueues nothing.  A
 *   launch failure returns SPEC_EHIP; spec_last_hip_error() names it.
 * - Data errors only the device can see never fault: they set bits in the
 *   per-request out_flags (SPEC_FLAG_*) and the request's outputs follow the
 *   documented fallback.
 * - Calls are re-entrant and thread-safe; calls that share output or
 *   workspace buffers must be ordered by the caller (same stream).
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 6

/* ---- return codes ---------------------------------------------------- */
#define SPEC_OK          0
#define SPEC_EINVAL     (-1)  /* null pointer, bad size or enum             */
#define SPEC_EWORKSPACE (-2)  /* workspace missing or smaller than needed   */
#define SPEC_EHIP       (-3)  /* a HIP launch or query failed               */

/* ---- logits element types --------------------------------------------- */
#define SPEC_F32  0
#define SPEC_BF16 1           /* upcast to fp32 exactly on load             */

/* ---- per-request out_flags bits ---------------------------------------- */
#define SPEC_FLAG_RESIDUAL_ZERO (1u << 5)  /* residual had no mass: sampled from p  */
#define SPEC_FLAG_BAD_TOKEN     (1u << 8)  /* a draft token outside [0, vocab): the
                                              slot is rejected                       */
#define SPEC_FLAG_BAD_LOGITS    (1u << 9)  /* a read row had NaN/+Inf, or no finite
                                              entry; its outputs are unspecified     */
#define SPEC_FLAG_CTX_OVERFLOW  (1u << 10) /* commit skipped: context capacity       */
#define SPEC_FLAG_BAD_LENGTH    (1u << 11) /* a length argument was clamped          */
#define SPEC_FLAG_RESIDUAL_LATE (1u << 12) /* the residual's published chunk sums did
                                              not all arrive within the bounded wait:
                                              the drawing workgroup summed the
                                              residual again itself (same result up
                                              to rounding order)                     */
#define SPEC_FLAG_BAD_FOREST    (1u << 13) /* a caller-built forest broke its rules
                                              (a parent not below its child, or a q
                                              outside [0, 1]): its rows are the
                                              anchor alone                           */

/* ---- slot flags (chain slots) ----------------------------------------- */
#define SPEC_SLOT_POINT_MASS 1u  /* verify as a point mass, q = delta_y         */
#define SPEC_SLOT_FROM_NGRAM 2u  /* the token came from the n-gram chain        */

/* ---- chosen-chain source ---------------------------------------------- */
#define SPEC_SRC_MODEL    0
#define SPEC_SRC_NGRAM    1
#define SPEC_SRC_MERGED   2   /* contains rule: n-gram chain, merged survivals */
#define SPEC_SRC_EXTENDED 3   /* extension policy: model chain + n-gram tail   */

/* ---- chain-selection policies ([HS] Section 4.3, Appendix H) ----------- */
#define SPEC_POLICY_PROPOSED    0  /* contains rule, then value rule at lambda */
#define SPEC_POLICY_NGRAM_FIRST 1  /* n-gram chain whenever it matched          */
#define SPEC_POLICY_EXTENSION   2  /* model chain; append n-gram tail if prefix */
#define SPEC_POLICY_MODEL_ONLY  3
#define SPEC_POLICY_NGRAM_ONLY  4

/* ---- allocation modes --------------------------------------------------- */
#define SPEC_ALLOC_CHAIN 0
#define SPEC_ALLOC_TREE  1

/* ---- operation ids for spec_workspace_bytes ------------------------------ */
#define SPEC_OP_NGRAM        0
#define SPEC_OP_ALLOCATE     1
#define SPEC_OP_VERIFY_CHAIN 2
#define SPEC_OP_VERIFY_TREE  3

/* Limits. */
#define SPEC_MAX_DRAFT   32   /* n-gram draft length, chain leading dim      */
#define SPEC_MAX_CAP   1024   /* n-gram comparison cap (copy_cap)            */
#define SPEC_MAX_FOLLOW_CTX 8 /* follower fallback context (follow_ctx)      */
#define SPEC_MAX_FOLLOWERS 1024 /* distinct followers a fallback step counts */
#define SPEC_MAX_ROWS    64   /* tree rows per request                       */
#define SPEC_MAX_FOREST 1024  /* tree candidates per request                 */
#define SPEC_MAX_VOCAB  8388608 /* logits per row                            */

/* ========================================================================
 * spec_ngram_draft -- prompt-lookup n-gram drafter ([HS] Section 4.1 "One
 * step", Section 4.2 match features; Algorithm 1, the NGRAMSCAN call).
 *
 * For query q its text x is ctx[req][0 .. ctx_len[req]) followed by
 * extra[q][0 .. extra_len[q]), with req = query_req ? query_req[q] : q.  Every
 * earlier end position j (j <= |x|-2) has a match length l_j, the number of
 * trailing tokens of x[..j] equal to the trailing tokens of x, compared up to
 * min(j+1, copy_cap).  Among positions with l_j >= n_min the best is the
 * longest, ties to the latest j; the runner-up is the next in that order.
 * Outputs: draft[q] = up to max_draft tokens after the best match (padded
 * with -1), draft_len[q], and feat[q] = (n, a, m, j) with
 * n = min(l_best, n_max), m = l_best if l_best >= n_max else 0, a = 1 if there
 * is no runner-up or it is followed by the same token, j = best end position
 * (-1 and zeros when nothing matched).  Integer only; deterministic.
 * Lengths outside [0, stride] are clamped.
 *
 * Follower fallback ([AS] Section 3.3, "N-gram candidates": the tree's
 * n-gram fill reads on along the earlier passage, or else takes the most
 * frequent follower of its last three tokens), on when follow_ctx = F > 0:
 * once the copy ends (the passage reaches the end of x, or nothing matched)
 * each further draft token is the most frequent follower, over x, of the
 * last F tokens of x ++ the draft so far (occurrences ending at p <= |x|-2,
 * follower x[p+1]); ties go to the follower seen latest; a context with no
 * follower or more than SPEC_MAX_FOLLOWERS distinct ones ends the draft.
 * draft_follow[q][k] = that follower's count (0 for copied tokens and past
 * the draft).  feat describes the copy only.
 * ======================================================================== */
typedef struct spec_ngram_args {
    int32_t bs;                  /* requests (rows of ctx)                        */
    int32_t nq;                  /* queries                                       */
    const int32_t* ctx;          /* device [bs, ctx_stride] token ids             */
    int64_t ctx_stride;          /* elements between request rows, >= 1          */
    const int32_t* ctx_len;      /* device [bs]                                   */
    const int32_t* query_req;    /* device [nq] or NULL (then nq <= bs)           */
    const int32_t* extra;        /* device [nq, extra_stride] or NULL             */
    int64_t extra_stride;        /* 0 when extra is NULL                          */
    const int32_t* extra_len;    /* device [nq] or NULL                           */
    int32_t n_min;               /* >= 1                                          */
    int32_t n_max;               /* >= n_min                                      */
    int32_t max_draft;           /* 1 .. SPEC_MAX_DRAFT                           */
    int32_t copy_cap;            /* n_min .. SPEC_MAX_CAP (256 on the pages)      */
    int32_t follow_ctx;          /* 0 (no fallback) .. SPEC_MAX_FOLLOW_CTX (3 for
                                    the tree's n-gram fill on the pages)          */
    int32_t* draft;              /* device [nq, max_draft]                        */
    int32_t* draft_len;          /* device [nq]                                   */
    int32_t* feat;               /* device [nq, 4]                                */
    int32_t* draft_follow;       /* device [nq, max_draft] or NULL: follower
                                    counts (follow_ctx > 0)                       */
    void* workspace;             /* device scratch                                */
    size_t workspace_bytes;
} spec_ngram_args;

/* ========================================================================
 * spec_allocate_budget
 *
 * Chain mode ([HS] Algorithm 1, Sections 4.2-4.4): per request, the n-gram
 * acceptance estimates (Eq. (1)),
 *   h_k = sigmoid(beta_k + w_pos(k)(n - n_ref) + delta a
 *                 + [n >= n_full](l_pos(k) + kappa_pos(k) ln(min(m, m_cap)/m_ref))),
 * the survivals S^g_k = prod h, S^d_k = prod c (c = model confidences), one
 * chosen chain per request by `policy` (proposed: contains rule, else value
 * rule V = sum_k max(S_k - lambda, 0) with ties to the n-gram chain, Eq. (3)),
 * and the batch-wide allocation of `budget` draft slots to the highest
 * survivals (ties: lower position, then lower request; keys are the
 * survivals rounded to fp32), so every request keeps a prefix.  Rows per
 * request = allocated slots + 1; row_base is their exclusive prefix sum.
 * Estimates, survivals and values are computed in fp64.
 *
 * Tree mode ([AS] Sections 2.2, 3.1, 3.3): the candidate forest of a drafter
 * block (P positions x Kc ranked candidates: the pick at p hangs from the pick
 * at p-1, siblings from the same parent) plus n-gram chains from the anchor
 * and each pick (a step equal to an existing child descends into it, else a
 * new node; no node deeper than depth_max); acceptance estimates by the form
 * of Eq. (6), q_j = w_node[j] / (w_none[parent] + sum of w_node over the
 * parent's children), Q = product of q along the path; the best rows_cap-1
 * candidates by Q (ties to the lower index) laid out depth-first (row 0 = the
 * anchor, children in index order).
 * A forest the caller built (forest_token != NULL; [AS] Section 3.1 takes any
 * drafter's candidate forest): node j's parent index lies in [0, j), node 0
 * is the anchor, and q_j in [0, 1] is its acceptance estimate given that its
 * parent is accepted.  Then Q_j = Q_parent q_j (fp64, Q = 1 at the anchor) and
 * the rows are chosen and laid out as above; block, the n-gram chains, the
 * weights and depth_max are not read (scores must be NULL).  A forest that
 * breaks a rule is flagged (SPEC_FLAG_BAD_FOREST) and keeps the anchor
 * alone; forest_n outside [1, c_max] is clamped (SPEC_FLAG_BAD_LENGTH).
 * ======================================================================== */
typedef struct spec_estimator {
    float beta[15];              /* per-position intercepts                       */
    float w_first, w_rest;       /* match-length weights                          */
    float delta;                 /* agreement weight                              */
    float l_first, l_rest;       /* full-match bonus                              */
    float k_first, k_rest;       /* copy-length weights                           */
    float n_ref;                 /* 5 on the pages                                */
    float n_full;                /* 15                                            */
    float m_ref;                 /* 15                                            */
    float m_cap;                 /* 256                                           */
} spec_estimator;

typedef struct spec_chain_alloc {
    int32_t bs;
    int32_t K;                   /* model chain length (7), 0..ld                 */
    int32_t ld;                  /* leading dim of chain outputs, max(K,L)..32    */
    const int32_t* model_tokens; /* device [bs, K]                                */
    const float* model_conf;     /* device [bs, K] confidences                    */
    int32_t conf_is_logit;       /* 1: model_conf are logits (c = sigmoid)        */
    const uint8_t* model_point_mass; /* device [bs] (1 = greedy drafting) or NULL = all 1 */
    const int32_t* ngram_draft;  /* device [bs, ngram_ld] (spec_ngram_draft)      */
    int32_t ngram_ld;            /* <= ld                                         */
    const int32_t* ngram_len;    /* device [bs]                                   */
    const int32_t* ngram_feat;   /* device [bs, 4]                                */
    spec_estimator est;
    float lambda;                /* slot price                                    */
    int32_t budget;              /* b*, verified draft slots for the batch, >= 0  */
    int32_t policy;              /* SPEC_POLICY_*                                 */
    int32_t* chain_tokens;       /* device [bs, ld], -1 padded                    */
    uint8_t* slot_flags;         /* device [bs, ld] SPEC_SLOT_*                   */
    int32_t* chain_len;          /* device [bs]                                   */
    int32_t* chain_src;          /* device [bs] SPEC_SRC_*                        */
    float* survival;             /* device [bs, ld] (0 past chain_len)            */
    int32_t* alloc_len;          /* device [bs] slots to verify (a chain prefix)  */
    int64_t* row_base;           /* device [bs]                                   */
    int32_t* total_rows;         /* device [1] = budget used + bs                 */
    uint32_t* out_flags;         /* device [bs], written (not OR-ed)              */
} spec_chain_alloc;

/* Acceptance estimates of the Eq. (6) form from its scores ([AS] Section 3.3,
 * "Form"): q_j = exp(s_j) / (1 + the sum of exp(s) over the parent's
 * candidates), the 1 being the explicit 'none' outcome, with
 *   pick:    s = a0 + a1 logit h + a2 logit sigma + psi + b_req
 *   sibling: s = a3 + a4 log r + a5 logit h + a6 logit sigma + psi + b_req
 *   n-gram:  s = logit p_src + w_bucket[bucket] + psi_ctx + b_req
 * with psi = psi_ctx + psi_depth[p] for a drafter candidate at position p.  A
 * drafter candidate an n-gram chain also proposes (agreed) adds
 * max(0, logit p_src) + w_agreed[proposal bucket][pick 0 / sibling 1]; one
 * whose parent has an n-gram proposal of another token (contradicted)
 * subtracts max(0, logit p_src) and adds w_contra[that proposal's evidence
 * class][pick 0 / sibling 1]; the largest such bucket or class counts.  An
 * n-gram node's evidence is its source's match length l (feature m, else n)
 * or, for a token of the follower fallback, its follower count l; class
 * e = min(7, floor(log2 l)); its bucket is 4 e + min(3, n-gram nodes above it
 * on its path), plus 32 for a follower token.  Probabilities are clamped to [1e-6, 1 - 1e-6]
 * before logit / log; everything in fp64.  With the prior a = (ln 2, 1, 0,
 * 0, 1, 0, 0) and zero weights a pick's estimate is h. */
typedef struct spec_tree_scores {
    double a[7];
    double w_bucket[64];         /* 0..31 copied tokens, 32..63 followers         */
    double w_agreed[64][2];
    double w_contra[8][2];
    double psi_depth[16];        /* by position p (p >= 15 uses 15)               */
    const float* h;              /* device [bs, P] confidence head per position   */
    const float* sigma;          /* device [bs, P] the pick's share               */
    const float* r_share;        /* device [bs, P, Kc] a sibling's share of its
                                    siblings' total (k >= 1)                      */
    const float* psi_ctx;        /* device [bs] context term                      */
    const float* b_req;          /* device [bs] per-request intercept             */
    const float* p_src;          /* device [bs] the n-gram source's precision     */
    const int32_t* ngram_feat;   /* device [bs*(P+1), 4] (n, a, m, j) of each
                                    chain's draft (spec_ngram_draft's feat)       */
} spec_tree_scores;

typedef struct spec_tree_alloc {
    int32_t bs;
    int32_t P;                   /* drafter block positions                      */
    int32_t Kc;                  /* ranked candidates per position               */
    const int32_t* block;        /* device [bs, P, Kc], rank 0 = the pick         */
    const int32_t* ngram_draft;  /* device [bs*(P+1), ngram_ld]: source s = 0 is
                                    the anchor, s = i the pick at position i      */
    int32_t ngram_ld;
    const int32_t* ngram_len;    /* device [bs*(P+1)]                             */
    const int32_t* ngram_follow; /* device [bs*(P+1), ngram_ld] follower counts of
                                    the chains' tokens (draft_follow), or NULL    */
    const float* w_node;         /* device [bs, c_max] > 0, by candidate index    */
    const float* w_none;         /* device [bs, c_max] > 0, 'none' of a parent    */
    const spec_tree_scores* scores; /* host, or NULL: with it the weights are
                                    exp(s) of the Eq. (6) scores (w_none = 1) and
                                    w_node / w_none are not read                  */
    int32_t c_max;               /* 1 + P*Kc .. SPEC_MAX_FOREST                   */
    int32_t depth_max;           /* >= 1 (32 on the pages)                        */
    int32_t rows_cap;            /* 1 .. SPEC_MAX_ROWS                            */
    int32_t* node_token;         /* device [bs, rows_cap] (row 0: -1)             */
    int32_t* parent_row;         /* device [bs, rows_cap] (row 0: -1)             */
    float* Q;                    /* device [bs, rows_cap]                         */
    int32_t* n_rows;             /* device [bs]                                   */
    int64_t* row_base;           /* device [bs] exclusive prefix sum of n_rows    */
    int32_t* total_rows;         /* device [1]                                    */
    int32_t* forest_count;       /* device [bs] candidates incl. the anchor       */
    float* s_curve;              /* device [bs, rows_cap] or NULL: S(n) for n = 1..
                                    rows_cap, the sum of Q over the first n - 1
                                    nodes of the best-first order ([AS] Section
                                    3.1; one walk down the order gives every n)   */
    uint32_t* out_flags;         /* device [bs], written                          */
    const int32_t* forest_token; /* device [bs, c_max] or NULL: a caller-built
                                    forest's tokens (node 0, the anchor: unread)  */
    const int32_t* forest_parent;/* device [bs, c_max] parent index, in [0, j)    */
    const float* forest_q;       /* device [bs, c_max] acceptance estimate of a
                                    node given its parent, in [0, 1]              */
    const int32_t* forest_n;     /* device [bs] nodes incl. the anchor, 1..c_max  */
} spec_tree_alloc;

typedef struct spec_alloc_args {
    int32_t mode;                /* SPEC_ALLOC_CHAIN or SPEC_ALLOC_TREE           */
    spec_chain_alloc chain;
    spec_tree_alloc tree;
    void* workspace;
    size_t workspace_bytes;
} spec_alloc_args;

/* ========================================================================
 * spec_verify_chain -- lossless verification of one chain per request
 * ([LS] Section 2.1 with the speculative-sampling rule that [HS] Section 2
 * cites; point-mass slots per [HS] Section 5.8 and Appendix H).
 *
 * Request r has b = n_slots[r] slots with tokens y_1..y_b.  Target row
 * row_base[r] + k (k = 0..b) scores slot k+1 (k = b is the bonus row); draft
 * row draft_row_base[r] + k scores slot k+1 for probabilistic slots.
 * T > 0: p = softmax(z/T), q = softmax(w/T) (q = delta_y for point-mass
 * slots); slot i is accepted iff u_accept[r][i] < p(y_i)/q(y_i) (fp64); at
 * the first rejection the correction is drawn from norm(max(0, p - q)), or
 * the bonus from p of row b when all pass, by inverse CDF in token order with
 * u_sample[r].  T = 0: accept iff y_i = argmax z (ties to the lowest id); the
 * correction / bonus is the argmax.  Out: out_tokens[r][0..out_num) = the
 * accepted tokens then the correction or bonus, out_num = accepted + 1,
 * out_p[r][i] / out_q[r][i] = p(y_{i+1}) / q(y_{i+1}) for every slot i < b
 * (q = 1 for point masses and at T = 0, where p is 1 or 0); out_p[r][b] = p of
 * the bonus row at the bonus token when every slot passed (1 at T = 0), else 0;
 * entries past them are 0.  out_flags is OR-ed (written with
 * write_flags).  If ctx is not NULL the
 * emitted tokens are appended to ctx[r] at ctx_len[r] (skipped and flagged if
 * ctx_len + out_num > ctx_cap).  n_slots outside [0, ld] are clamped.
 * With ngram_draft (which needs ctx), the next step's n-gram draft of every
 * request ([HS] Section 4.1 "One step": scan the request's own text after the
 * commit) is computed in the same launch, over the committed context: the
 * outputs equal spec_ngram_draft's with query q = request q over ctx and the
 * new lengths, and n-gram parameters as documented there.
 * ======================================================================== */
typedef struct spec_verify_args {
    int32_t bs;
    int32_t vocab;
    float temperature;           /* >= 0; 0 = greedy                              */
    const void* logits;          /* device target rows                            */
    int32_t dtype;               /* SPEC_F32 / SPEC_BF16                          */
    int64_t row_stride;          /* elements between rows, >= vocab               */
    const int64_t* row_base;     /* device [bs]                                   */
    int64_t n_logit_rows;        /* rows in the logits buffer: a row index outside
                                    [0, n_logit_rows) is never read (flagged)     */
    const void* draft_logits;    /* device draft rows; NULL if every slot is a
                                    point mass or T = 0                           */
    int32_t draft_dtype;
    int64_t draft_row_stride;
    const int64_t* draft_row_base; /* device [bs] or NULL with draft_logits       */
    int64_t n_draft_rows;        /* rows in the draft buffer                      */
    const int32_t* tokens;       /* device [bs, ld]                               */
    const uint8_t* slot_flags;   /* device [bs, ld] or NULL = all point masses    */
    int32_t ld;                  /* 1 .. SPEC_MAX_DRAFT                           */
    const int32_t* n_slots;      /* device [bs]                                   */
    int32_t max_slots;           /* optional host bound of the sum of the clamped
                                    n_slots (e.g. the allocation budget); 0 = bs*ld.
                                    Sizes the row-statistics grid only: a bound
                                    that is too small costs speed, not results   */
    const float* u_accept;       /* device [bs, ld] uniforms in [0,1)             */
    const float* u_sample;       /* device [bs]                                   */
    int32_t rng;                 /* 1: the call draws its uniforms itself and
                                    u_accept / u_sample may be NULL: uniform k of
                                    request r is word k mod 4 of Philox4x32-10
                                    (Salmon et al., SC'11) with counter (k / 4, r,
                                    rng_offset low, high) and key rng_seed (low,
                                    high), as (word >> 8) 2^-24; u_accept[r][i] is
                                    uniform i, u_sample[r] uniform SPEC_MAX_DRAFT */
    uint64_t rng_seed;
    uint64_t rng_offset;         /* e.g. the step number                          */
    int32_t* out_tokens;         /* device [bs, ld+1], -1 padded                  */
    int32_t* out_num;            /* device [bs]                                   */
    int32_t* out_accepted;       /* device [bs]                                   */
    float* out_p;                /* device [bs, ld + 1] or NULL                   */
    float* out_q;                /* device [bs, ld] or NULL                       */
    uint32_t* out_flags;         /* device [bs], OR-ed (see write_flags)          */
    int32_t write_flags;         /* 1: out_flags[r] is written with this call's
                                    flags instead (no zeroing needed before)      */
    int32_t* out_accept_hist;    /* optional device [ld + 1]: entry a is increased
                                    by the requests that accepted a drafts (the
                                    acceptance length distribution; the prefix
                                    advances by a + 1, [LS] Section 2.1)         */
    int32_t* ctx;                /* optional commit: device [bs, ctx_stride]      */
    int64_t ctx_stride;
    int32_t* ctx_len;            /* device [bs]                                   */
    int32_t* ctx_len_out;        /* device [bs] or NULL: new lengths go here and
                                    ctx_len is left as it was (NULL = in place)   */
    int32_t ctx_cap;             /* <= ctx_stride                                 */
    int32_t* ngram_draft;        /* optional next n-gram draft: device
                                    [bs, ngram_max_draft] or NULL (none)          */
    int32_t* ngram_draft_len;    /* device [bs]                                   */
    int32_t* ngram_feat;         /* device [bs, 4]: (n, a, m, j)                  */
    int32_t ngram_n_min;         /* as n_min, n_max, max_draft and copy_cap of    */
    int32_t ngram_n_max;         /* spec_ngram_args                               */
    int32_t ngram_max_draft;
    int32_t ngram_copy_cap;
    int32_t residual_wait;       /* polls of one published residual chunk sum before
                                    the drawing workgroup gives up on it and sums
                                    the residual itself (SPEC_FLAG_RESIDUAL_LATE);
                                    0 = 2^20, < 0 = give up at once (a test of the
                                    fallback: the sums are then never waited for) */
    void* prof_begin;            /* optional hipEvent_t pair (created with timing) */
    void* prof_end;              /* attached to the row-statistics kernel's own
                                    dispatch: begin = its start, end = its end    */
    void* workspace;
    size_t workspace_bytes;
} spec_verify_args;

/* ========================================================================
 * spec_verify_tree -- greedy tree verification ([AS] Section 2.2): starting
 * at the anchor (row 0), a child is accepted when its token equals the
 * argmax (ties to the lowest id) of its parent's row; the accepted nodes form
 * one path; out_tokens = the path's tokens then the argmax at its last node,
 * out_num = path length + 1, out_path_rows = the rows of the anchor and the
 * accepted nodes.  T = 0 only.  Optional commit as in spec_verify_chain.
 * ======================================================================== */
typedef struct spec_tree_verify_args {
    int32_t bs;
    int32_t vocab;
    int32_t rows_max;            /* leading dim of the tree arrays, <= SPEC_MAX_ROWS */
    const void* logits;          /* device rows                                   */
    int32_t dtype;
    int64_t row_stride;
    const int64_t* row_base;     /* device [bs]                                   */
    int64_t n_logit_rows;        /* rows in the logits buffer (bounds)            */
    const int32_t* node_token;   /* device [bs, rows_max]                         */
    const int32_t* parent_row;   /* device [bs, rows_max]                         */
    const int32_t* n_rows;       /* device [bs], 1..rows_max (clamped)            */
    int32_t* out_tokens;         /* device [bs, rows_max]                         */
    int32_t* out_num;            /* device [bs]                                   */
    int32_t* out_path_rows;      /* device [bs, rows_max]                         */
    int32_t* out_argmax;         /* device [bs, rows_max] or NULL                 */
    uint32_t* out_flags;         /* device [bs], OR-ed                            */
    int32_t* ctx;
    int64_t ctx_stride;
    int32_t* ctx_len;
    int32_t* ctx_len_out;        /* as in spec_verify_args                        */
    int32_t ctx_cap;
    void* prof_begin;            /* optional hipEvent_t pair (as in spec_verify_args) */
    void* prof_end;
    void* workspace;
    size_t workspace_bytes;
} spec_tree_verify_args;

/* ========================================================================
 * spec_size_budget -- budget sizing and slot price, host arithmetic ([HS]
 * Section 2 "Adaptive verification" and "Asynchronous scheduling", Section
 * 4.3 "Slot price" Eq. (2), Section 4.4, Appendix F with Eq. (4)).
 *
 * survival: host [n] survivals of the batch's chosen chains (the copy of the
 * allocation's `survival` output a step earlier; entries <= 0 or padding add
 * nothing).  A(b) = n_requests + (the b largest survivals) is the expected
 * number of emitted tokens, C(b) the step cost and G(b) = A(b)/C(b) the
 * goodput.  C(b) = c0 + p b; when graph_limit > 0 and n_tokens + b exceeds it
 * the step runs eagerly and C(b) = max(c0 + p b, eager[n_tokens + b -
 * graph_limit - 1]) (Eq. (4)); a b beyond that table cannot run.  Out:
 * *b_star = the b in [0, b_max] (b_max <= 0: n) with the largest G (ties to
 * the smaller b), *lambda = G(b*) p (Eq. (2)), *goodput = G(b*) (or NULL);
 * with goodput_curve (host [1 + min(n, b_max)], b_max <= 0 meaning n, or
 * NULL) G(b) for every b (-1 where b cannot run).  All in double over the survivals in descending order.
 * Host memory only; no device work.  SPEC_EINVAL for bad arguments.
 * ======================================================================== */
typedef struct spec_cost_model {
    double c0;                   /* base step cost C0 (any unit of time), > 0     */
    double p;                    /* cost of one draft slot, >= 0                  */
    int32_t graph_limit;         /* tokens a captured step holds; 0 = no limit    */
    int32_t n_tokens;            /* N: the step's non-draft tokens                */
    const double* eager;         /* host [n_eager]: eager[k] = T(graph_limit + 1 + k)
                                    + C_KV, the profiled eager step costs         */
    int32_t n_eager;
} spec_cost_model;

int spec_size_budget(const float* survival, int64_t n, int32_t n_requests, const spec_cost_model* cost,
                     int32_t b_max, int32_t* b_star, double* lambda, double* goodput, double* goodput_curve);

int spec_ngram_draft(const spec_ngram_args* args, void* stream);
int spec_allocate_budget(const spec_alloc_args* args, void* stream);
int spec_verify_chain(const spec_verify_args* args, void* stream);
int spec_verify_tree(const spec_tree_verify_args* args, void* stream);

/* ========================================================================
 * spec_verify_chain_noalloc -- spec_verify_chain for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs and kernels;
 * args->workspace and workspace_bytes are ignored: the scratch comes from one
 * array of SPEC_NOALLOC_SCRATCH_BYTES per device inside the library, which
 * the device holds from the first call until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Returns SPEC_EWORKSPACE when the call needs more scratch than that (see
 * spec_workspace_bytes(SPEC_OP_VERIFY_CHAIN, args)), else as
 * spec_verify_chain.  All calls on one device share its array: calls that
 * may overlap on a device (other streams, other threads) race and must be
 * ordered by the caller; consecutive calls on one stream are safe.
 * ======================================================================== */
#define SPEC_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_chain_noalloc(const spec_verify_args* args, void* stream);

/* Workspace bytes the call with these arguments needs (0 = none); a host-only
 * query that reads sizes from args and never touches device memory. */
size_t spec_workspace_bytes(int op, const void* args);
const char* spec_strerror(int code);
const char* spec_last_hip_error(void);   /* thread-local, last SPEC_EHIP cause */
int spec_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_H */
