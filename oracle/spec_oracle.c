/*
 * spec_oracle.c -- plain, slow, fp64 CPU oracle of the speculative-decoding
 * step (n-gram draft, acceptance estimates and survivals, chain selection,
 * budget allocation, chain verification by rejection sampling, tree build and
 * greedy tree verification, commit).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the HIP path; the two meet only on the seeded inputs.
 *
 * Sources (titles of the pages the method is described on):
 *   [HS] "Hybrid Spark: Adaptive Speculative Decoding That Lets the Content
 *        Choose the Drafter"
 *   [AS] "AdaSpark: Adaptive DSpark with Online Learning for Tree Verification
 *        and N-gram Fill"
 *   [LS] "Efficient speculative decoding with a fixed-cost parallel drafter"
 *        (LongSpark), Section 2.1 (the verification round)
 *
 * Every decision that floating point takes is taken here in the precision the
 * HIP kernels take it in (documented per function); the oracle additionally
 * flags near ties so that tests can excuse them.
 *
 * Parity pins: every function below is pinned by a test (printed values,
 * closed forms, brute force or Monte Carlo); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Per-request flag bits (the same meanings as the library's out_flags). */
#define OF_ACCEPT_NEAR   (1u << 0)  /* |u - rho| < 1e-6 at an evaluated slot    */
#define OF_SAMPLE_NEAR   (1u << 1)  /* u'W within 1e-6 W of the chosen CDF bound */
#define OF_SELECT_NEAR   (1u << 2)  /* |V_g - V_d| <= 1e-6 max(1, V_d)           */
#define OF_ALLOC_NEAR    (1u << 3)  /* a slot near the allocation cut            */
#define OF_TREE_NEAR     (1u << 4)  /* a node near the best-first cut            */
#define OF_RESIDUAL_ZERO (1u << 5)  /* residual had zero mass; sampled from p    */
#define OF_BAD_TOKEN     (1u << 8)  /* a draft token outside [0, V)              */
#define OF_BAD_LOGITS    (1u << 9)  /* a row with non-finite statistics          */
#define OF_CTX_OVERFLOW  (1u << 10) /* commit would exceed the context capacity  */
#define OF_BAD_LENGTH    (1u << 11) /* a length argument was clamped             */
#define OF_BAD_FOREST    (1u << 13) /* a given forest broke its rules            */

#define NEAR_EPS 1e-6

/* A planted mistake, compiled in only by the tests that show the Monte Carlo
 * losslessness checks detect one: 1 = sample the correction from p instead of
 * the residual; 2 = accept with probability p(y) ignoring q; 3 = verify the
 * extension policy's n-gram tail against q instead of as point masses; 4 =
 * n-gram-first keeps the drafter's chain when its first sampled token is 0
 * (a choice that reads the drafter's samples).  0 = correct. */
#ifndef SPEC_ORACLE_MUTATION
#define SPEC_ORACLE_MUTATION 0
#endif

/* Chain sources and slot flags. */
#define SRC_MODEL 0
#define SRC_NGRAM 1
#define SRC_MERGED 2
#define SRC_EXTENDED 3
#define SLOT_POINT_MASS 1u
#define SLOT_FROM_NGRAM 2u

/* Selection policies ([HS] Section 4.3 and Appendix H). */
#define POL_PROPOSED 0
#define POL_NGRAM_FIRST 1
#define POL_EXTENSION 2
#define POL_MODEL_ONLY 3
#define POL_NGRAM_ONLY 4

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* A logits element as fp64: dtype 0 = fp32, 1 = bf16 stored as uint16. */
static double logit_at(const void* base, int dtype, int64_t i)
{
    if (dtype == 0) return (double)((const float*)base)[i];
    uint32_t b = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return (double)f;
}

/* ======================================================================
 * N-gram scan.  [HS] Section 4.1 ("One step") and Section 4.2 (match
 * features); Algorithm 1, the NGRAMSCAN call.
 *
 * For the query text x[0..T-1], every earlier end position j (j <= T-2) has
 * a match length l_j: the number of trailing tokens of x[..j] that equal the
 * trailing tokens of the whole text, compared up to min(j+1, cap).  Positions
 * with l_j >= n_min are matches.  The best match is the longest one, ties
 * going to the most recent (readings: the longer match is preferred, and
 * recency breaks ties); the runner-up is the next one in the same order.  Features:
 *   n = min(l_best, n_max); full = l_best >= n_max; m = l_best if full else 0;
 *   a = 1 if there is no runner-up or it predicts the same next token.
 * The draft is the up-to-max_draft tokens after the best match.
 * ====================================================================== */
/* ======================================================================
 * N-gram fill's fallback.  [AS] Section 3.3, "N-gram candidates": a chain
 * reads on along the earlier passage, or else takes the most frequent
 * follower of its last three tokens (the context length F is a parameter).
 *
 * Readings: the fallback takes over for every position after the copy ends
 * (the passage reaches the end of the text, or there was no match), one
 * token at a time.  The context is the last F tokens of the text followed by
 * the chain so far; its occurrences are counted in the text only, each with
 * its follower inside the text.  The most frequent follower wins, ties going
 * to the follower seen latest (the later-wins order of the copy rule).  A
 * context with no follower, or with more than ORACLE_MAX_FOLLOWERS distinct
 * followers, ends the chain.  follow[k] is the count of the winning follower
 * at position k (0 for a copied token).
 * ====================================================================== */
#define ORACLE_MAX_FOLLOWERS 1024

static void follower_fill(const int32_t* x, int64_t T, int F, int max_draft, int32_t* draft, int64_t* len,
                          int32_t* follow)
{
    int32_t ftok[ORACLE_MAX_FOLLOWERS], fcnt[ORACLE_MAX_FOLLOWERS];
    int64_t flast[ORACLE_MAX_FOLLOWERS];
    int32_t c[64];
    if (F > 64) return;
    while (*len < max_draft && T + *len >= F) {
        for (int i = 0; i < F; ++i) {           /* position T + len - F + i of text ++ chain */
            int64_t q = T + *len - F + i;
            c[i] = q < T ? x[q] : draft[q - T];
        }
        int nd = 0, over = 0;
        for (int64_t p = F - 1; p + 1 < T; ++p) {
            int i = 0;
            while (i < F && x[p - (F - 1) + i] == c[i]) ++i;
            if (i < F) continue;
            int32_t f = x[p + 1];
            int k = 0;
            while (k < nd && ftok[k] != f) ++k;
            if (k < nd) { ++fcnt[k]; flast[k] = p; continue; }
            if (nd == ORACLE_MAX_FOLLOWERS) { over = 1; continue; }
            ftok[nd] = f; fcnt[nd] = 1; flast[nd] = p; ++nd;
        }
        if (over || nd == 0) break;
        int b = 0;
        for (int k = 1; k < nd; ++k)
            if (fcnt[k] > fcnt[b] || (fcnt[k] == fcnt[b] && flast[k] > flast[b])) b = k;
        draft[*len] = ftok[b];
        follow[*len] = fcnt[b];
        ++*len;
    }
}

static void ngram_one(const int32_t* x, int64_t T, int n_min, int n_max, int max_draft, int cap, int follow_ctx,
                      int32_t* draft, int32_t* draft_len, int32_t* feat, int32_t* follow)
{
    for (int k = 0; k < max_draft; ++k) follow[k] = 0;
    int64_t best_j = -1, best_l = 0, ru_j = -1, ru_l = 0;
    for (int64_t j = 0; j + 1 < T; ++j) {
        int64_t lim = (j + 1 < cap) ? j + 1 : cap;
        int64_t l = 0;
        while (l < lim && x[j - l] == x[T - 1 - l]) ++l;
        if (l < n_min) continue;
        /* order: longer first, then later position (j grows, so later wins ties) */
        if (l > best_l || (l == best_l && j > best_j)) {
            ru_j = best_j; ru_l = best_l;
            best_j = j; best_l = l;
        } else if (l > ru_l || (l == ru_l && j > ru_j)) {
            ru_j = j; ru_l = l;
        }
    }
    for (int k = 0; k < max_draft; ++k) draft[k] = -1;
    if (best_j < 0) {
        int64_t len = 0;
        if (follow_ctx > 0) follower_fill(x, T, follow_ctx, max_draft, draft, &len, follow);
        *draft_len = (int32_t)len;
        feat[0] = 0; feat[1] = 0; feat[2] = 0; feat[3] = -1;
        return;
    }
    int64_t n = best_l < n_max ? best_l : n_max;
    int full = best_l >= n_max;
    int a = (ru_j < 0) || (x[ru_j + 1] == x[best_j + 1]);
    int64_t avail = T - 1 - best_j;
    int64_t len = avail < max_draft ? avail : max_draft;
    for (int64_t k = 0; k < len; ++k) draft[k] = x[best_j + 1 + k];
    if (follow_ctx > 0) follower_fill(x, T, follow_ctx, max_draft, draft, &len, follow);
    *draft_len = (int32_t)len;
    feat[0] = (int32_t)n;
    feat[1] = a;
    feat[2] = full ? (int32_t)best_l : 0;
    feat[3] = (int32_t)best_j;
}

/* Batch form: query q reads request req = query_req ? query_req[q] : q; its
 * text is ctx[req][0..ctx_len[req]) followed by extra[q][0..extra_len[q]). */
void oracle_ngram_draft(int nq, const int32_t* ctx, int64_t ctx_stride, const int32_t* ctx_len,
                        const int32_t* query_req, const int32_t* extra, int64_t extra_stride,
                        const int32_t* extra_len, int n_min, int n_max, int max_draft, int cap, int follow_ctx,
                        int32_t* draft, int32_t* draft_len, int32_t* feat, int32_t* follow)
{
    int32_t* fl_tmp = follow ? NULL : (int32_t*)malloc(sizeof(int32_t) * (size_t)max_draft);
    for (int q = 0; q < nq; ++q) {
        int req = query_req ? query_req[q] : q;
        int64_t tl = ctx_len[req];
        int64_t el = (extra && extra_len) ? extra_len[q] : 0;
        int32_t* x = (int32_t*)malloc(sizeof(int32_t) * (size_t)(tl + el + 1));
        memcpy(x, ctx + (int64_t)req * ctx_stride, sizeof(int32_t) * (size_t)tl);
        if (el) memcpy(x + tl, extra + (int64_t)q * extra_stride, sizeof(int32_t) * (size_t)el);
        ngram_one(x, tl + el, n_min, n_max, max_draft, cap, follow_ctx,
                  draft + (int64_t)q * max_draft, draft_len + q, feat + 4 * (int64_t)q,
                  follow ? follow + (int64_t)q * max_draft : fl_tmp);
        free(x);
    }
    free(fl_tmp);
}

/* ======================================================================
 * Acceptance estimate of n-gram draft position k (1-based).
 * [HS] Section 4.2, Eq. (1):
 *   h_k = sigma(beta_k + w_pos(k) (n - n_ref) + delta a
 *               + [n >= n_full] (l_pos(k) + kappa_pos(k) ln(min(m, m_cap) / m_ref)))
 * with pos(k) = first iff k = 1 (positions past 15, beyond the pages'
 * chains, reuse beta_15).  The copy term's garbled form is read as
 * ln(min(m,256)/15): under this reading a copy capped at 256 tokens is
 * worth kappa_first ln(256/15), about 5.7 logits, the size Appendix D
 * gives for it.  m >= 1 whenever the
 * term applies in consistent settings; the clamp only guards others.
 * ====================================================================== */
typedef struct {
    double beta[15];
    double w_first, w_rest, delta, l_first, l_rest, k_first, k_rest;
    double n_ref, n_full, m_ref, m_cap;
} oracle_estimator;

double oracle_estimate_logit(const oracle_estimator* e, int k, int n, int a, int m)
{
    int first = (k == 1);
    /* positions past the fifteenth share the last intercept */
    double z = e->beta[(k <= 15 ? k : 15) - 1] + (first ? e->w_first : e->w_rest) * ((double)n - e->n_ref)
             + e->delta * (double)a;
    if ((double)n >= e->n_full) {
        double mm = (double)m;
        if (mm < 1.0) mm = 1.0;
        if (mm > e->m_cap) mm = e->m_cap;
        z += (first ? e->l_first : e->l_rest) + (first ? e->k_first : e->k_rest) * log(mm / e->m_ref);
    }
    return z;
}

void oracle_estimate(const oracle_estimator* e, int n, int a, int m, int len, double* h)
{
    for (int k = 1; k <= len; ++k) h[k - 1] = sigmoid(oracle_estimate_logit(e, k, n, a, m));
}

/* Survivals as running products, S_k = prod_{j<=k} alpha_j ([HS] Section 2
 * and Algorithm 1, the survival lines). */
void oracle_survival(const double* alpha, int len, double* S)
{
    double s = 1.0;
    for (int k = 0; k < len; ++k) { s *= alpha[k]; S[k] = s; }
}

/* Chain value V = sum_k max(S_k - lambda, 0), [HS] Section 4.3, Eq. (3). */
double oracle_chain_value(const double* S, int len, double lambda)
{
    double v = 0.0;
    for (int k = 0; k < len; ++k) v += (S[k] > lambda) ? (S[k] - lambda) : 0.0;
    return v;
}

/* ======================================================================
 * Chain selection for one request.  [HS] Algorithm 1 and Section 4.3:
 *   contains rule: |g| > K and g_1..K = d  ->  keep g; S_k = max(S^g_k, S^d_k)
 *     for k <= K and S_k = S_{k-1} h_k after it (Algorithm 1 extends the
 *     merged prefix with the n-gram estimates);
 *   value rule: g matched and V(S^g) >= V(S^d) -> keep g (ties to n-gram);
 *   otherwise keep d.
 * Policies of Section 4.5 / Appendix H: n-gram-first keeps g whenever it
 * matched; extension keeps d and appends g's tail when d is a prefix of g
 * (tail survivals continue from S^d_K, tail slots are point masses).
 * Slot flags: n-gram slots are point masses; model slots are point masses
 * iff the model drafts greedily.  Values are compared in fp64.
 * Returns the chain length; *near is set when the value rule was a near tie.
 * ====================================================================== */
int oracle_select(int K, const int32_t* d, const double* c, int dlen,
                  const int32_t* g, const double* h, int glen,
                  double lambda, int policy, int model_point_mass, int ld,
                  int32_t* out_tok, uint8_t* out_flag, double* out_S, int32_t* out_src, int* near)
{
    double Sd[64], Sg[64];
    oracle_survival(c, dlen, Sd);
    oracle_survival(h, glen, Sg);
    *near = 0;
    int prefix = (glen > K && dlen == K);
    for (int i = 0; prefix && i < K; ++i) prefix = (g[i] == d[i]);
    uint8_t mfl = model_point_mass ? SLOT_POINT_MASS : 0;
    uint8_t gfl = SLOT_POINT_MASS | SLOT_FROM_NGRAM;
    int use = SRC_MODEL;  /* which chain */
    switch (policy) {
    case POL_PROPOSED:
        if (prefix) use = SRC_MERGED;
        else if (glen >= 1) {
            double vg = oracle_chain_value(Sg, glen, lambda);
            double vd = oracle_chain_value(Sd, dlen, lambda);
            double den = vd > 1.0 ? vd : 1.0;
            if (fabs(vg - vd) <= NEAR_EPS * den) *near = 1;
            use = (vg >= vd) ? SRC_NGRAM : SRC_MODEL;
        }
        break;
    case POL_NGRAM_FIRST:
        use = (glen >= 1) ? SRC_NGRAM : SRC_MODEL;
        if (SPEC_ORACLE_MUTATION == 4 && dlen >= 1 && d[0] == 0) use = SRC_MODEL;
        break;
    case POL_EXTENSION: use = prefix ? SRC_EXTENDED : SRC_MODEL; break;
    case POL_MODEL_ONLY: use = SRC_MODEL; break;
    case POL_NGRAM_ONLY: use = SRC_NGRAM; break;
    default: use = SRC_MODEL;
    }
    int len = 0;
    if (use == SRC_MODEL) {
        for (int k = 0; k < dlen; ++k) { out_tok[k] = d[k]; out_flag[k] = mfl; out_S[k] = Sd[k]; }
        len = dlen;
    } else if (use == SRC_NGRAM) {
        for (int k = 0; k < glen; ++k) { out_tok[k] = g[k]; out_flag[k] = gfl; out_S[k] = Sg[k]; }
        len = glen;
    } else if (use == SRC_MERGED) {
        for (int k = 0; k < glen; ++k) {
            out_tok[k] = g[k];
            out_flag[k] = gfl;
            if (k < K) out_S[k] = Sg[k] > Sd[k] ? Sg[k] : Sd[k];
            else out_S[k] = out_S[k - 1] * h[k];
        }
        len = glen;
    } else { /* SRC_EXTENDED */
        for (int k = 0; k < glen; ++k) {
            out_tok[k] = g[k];
            if (k < K) { out_flag[k] = mfl; out_S[k] = Sd[k]; }
            else { out_flag[k] = SPEC_ORACLE_MUTATION == 3 ? mfl : gfl; out_S[k] = out_S[k - 1] * h[k]; }
        }
        len = glen;
    }
    for (int k = len; k < ld; ++k) { out_tok[k] = -1; out_flag[k] = 0; out_S[k] = 0.0; }
    *out_src = use;
    return len;
}

/* ======================================================================
 * Verification-budget allocation.  [HS] Section 2 ("Adaptive verification")
 * and Algorithm 1, the AV line: the b* (request, position) slots with the
 * highest survival are verified; each request keeps a prefix of its chain.
 * Order: S descending, then position ascending, then request ascending
 * (reading: the pages give no tie rule; position-first keeps prefixes).  The
 * comparison is taken on S rounded to fp32, the precision of the kernel's
 * ranking keys.  Rows per request = allocated slots + 1 (the bonus or
 * correction row); row_base is the exclusive prefix sum of the rows.
 * A request is flagged when one of its slots and a slot on the other side of
 * the cut differ in fp64 by 0 < |dS| <= 1e-6 S.
 * ====================================================================== */
typedef struct { float s; double s64; int k; int r; } slot_t;

static int slot_cmp(const void* pa, const void* pb)
{
    const slot_t* a = (const slot_t*)pa;
    const slot_t* b = (const slot_t*)pb;
    if (a->s != b->s) return a->s > b->s ? -1 : 1;
    if (a->k != b->k) return a->k < b->k ? -1 : 1;
    if (a->r != b->r) return a->r < b->r ? -1 : 1;
    return 0;
}

void oracle_allocate(int bs, int ld, const int32_t* len, const double* S, int budget,
                     int32_t* alloc_len, int64_t* row_base, int32_t* total_rows, uint32_t* flags)
{
    int64_t n = 0;
    for (int r = 0; r < bs; ++r) n += len[r];
    slot_t* v = (slot_t*)malloc(sizeof(slot_t) * (size_t)(n > 0 ? n : 1));
    int64_t i = 0;
    for (int r = 0; r < bs; ++r)
        for (int k = 0; k < len[r]; ++k) {
            v[i].s64 = S[(int64_t)r * ld + k];
            v[i].s = (float)v[i].s64;
            v[i].k = k; v[i].r = r; ++i;
        }
    qsort(v, (size_t)n, sizeof(slot_t), slot_cmp);
    int64_t take = budget < n ? budget : n;
    for (int r = 0; r < bs; ++r) alloc_len[r] = 0;
    for (int64_t t = 0; t < take; ++t) alloc_len[v[t].r]++;
    /* near ties across the cut */
    for (int64_t a = 0; a < take; ++a)
        for (int64_t b = take; b < n; ++b) {
            double ds = fabs(v[a].s64 - v[b].s64);
            double ref = v[a].s64 > v[b].s64 ? v[a].s64 : v[b].s64;
            if (ds > 0.0 && ds <= NEAR_EPS * ref) {
                flags[v[a].r] |= OF_ALLOC_NEAR;
                flags[v[b].r] |= OF_ALLOC_NEAR;
            }
        }
    int64_t base = 0;
    for (int r = 0; r < bs; ++r) { row_base[r] = base; base += alloc_len[r] + 1; }
    *total_rows = (int32_t)base;
    free(v);
}

/* ======================================================================
 * Counter-based uniforms: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11).  A round multiplies
 * counter words 0 and 2 by M0 and M1 into 64-bit products and forms the new
 * counter (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0));
 * the key is bumped by the Weyl constants between rounds.  Philox4x64-10 is
 * the same with 64-bit words and its own constants (kept here so that the
 * round structure can be checked against a library generator).
 *
 * The step's uniforms (the mapping the verifier uses when it draws its own):
 * for request r at step `offset` with key `seed`, block j is
 * Philox4x32-10(counter = (j, r, offset_lo, offset_hi), key = (seed_lo,
 * seed_hi)); uniform k is word k mod 4 of block k / 4 as (w >> 8) 2^-24 in
 * [0, 1); u_accept[r][i] = uniform i, u_sample[r] = uniform 32.
 * ====================================================================== */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k[0];
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k[1];
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
        if (round < 9) { k[0] += 0x9E3779B9u; k[1] += 0xBB67AE85u; }
    }
    for (int i = 0; i < 4; ++i) out[i] = c[i];
}

static void mulhilo64(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo)
{
    unsigned __int128 p = (unsigned __int128)a * b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void oracle_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    uint64_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint64_t k[2] = {key_in[0], key_in[1]};
    for (int round = 0; round < 10; ++round) {
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(0xD2E7470EE14C6C93ull, c[0], &hi0, &lo0);
        mulhilo64(0xCA5A826395121157ull, c[2], &hi1, &lo1);
        uint64_t n0 = hi1 ^ c[1] ^ k[0], n2 = hi0 ^ c[3] ^ k[1];
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        if (round < 9) { k[0] += 0x9E3779B97F4A7C15ull; k[1] += 0xBB67AE8584CAA73Bull; }
    }
    for (int i = 0; i < 4; ++i) out[i] = c[i];
}

void oracle_step_uniforms(int bs, int ld, uint64_t seed, uint64_t offset, float* u_acc, float* u_smp)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int r = 0; r < bs; ++r) {
        float u[36];
        for (int j = 0; j < 9; ++j) {
            const uint32_t ctr[4] = {(uint32_t)j, (uint32_t)r, (uint32_t)offset, (uint32_t)(offset >> 32)};
            uint32_t w[4];
            oracle_philox4x32_10(ctr, key, w);
            for (int q = 0; q < 4; ++q) u[4 * j + q] = (float)((double)(w[q] >> 8) / 16777216.0);
        }
        for (int i = 0; i < ld; ++i) u_acc[(int64_t)r * ld + i] = u[i];
        u_smp[r] = u[32];
    }
}

/* ======================================================================
 * Budget sizing and slot price (host arithmetic).  [HS] Section 2, "Adaptive
 * verification": the budget b is the number of draft slots verified in one
 * pass; A(b) = B + (the b largest survivals of the batch) is the expected
 * number of emitted tokens of B requests, C(b) the step cost, and the budget
 * b* maximises the goodput G(b) = A(b) / C(b).  Appendix F: C(b) = C0 + p b;
 * above the graph capture limit (N + b > graph_limit tokens, N = the step's
 * non-draft tokens) the step runs eagerly and Eq. (4) gives
 * C(b) = max(C0 + p b, T(N + b) + C_KV), with the profiled eager costs
 * eager[k] = T(graph_limit + 1 + k) + C_KV; a b past the table cannot run.
 * Section 4.3, Eq. (2): the slot price is lambda = G(b*) p.  Ties of G go to
 * the smaller b.  All in fp64 over the survivals sorted in descending order.
 * ====================================================================== */
typedef struct {
    double c0, p;
    int32_t graph_limit;   /* 0 = no limit */
    int32_t n_tokens;      /* N */
    const double* eager;   /* [n_eager] */
    int32_t n_eager;
} oracle_cost;

/* C(b), or a negative value when b cannot run. */
double oracle_step_cost(const oracle_cost* cm, int b)
{
    double c = cm->c0 + cm->p * (double)b;
    if (cm->graph_limit > 0 && (int64_t)cm->n_tokens + b > cm->graph_limit) {
        int64_t k = (int64_t)cm->n_tokens + b - cm->graph_limit - 1;
        if (k >= cm->n_eager) return -1.0;
        if (cm->eager[k] > c) c = cm->eager[k];
    }
    return c;
}

static int desc_double(const void* pa, const void* pb)
{
    double a = *(const double*)pa, b = *(const double*)pb;
    return (a < b) - (a > b);
}

/* G(b) for every b in [0, b_max] (G[b] < 0: b cannot run); returns b*. */
int oracle_size_budget(const float* S, int n, int B, const oracle_cost* cm, int b_max, double* G, double* lambda)
{
    double* v = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) v[i] = S[i] > 0.0f ? (double)S[i] : 0.0;
    qsort(v, (size_t)n, sizeof(double), desc_double);
    if (b_max > n) b_max = n;
    double A = (double)B;
    int best = -1;
    for (int b = 0; b <= b_max; ++b) {
        if (b > 0) A += v[b - 1];
        double c = oracle_step_cost(cm, b);
        G[b] = c > 0.0 ? A / c : -1.0;
        if (G[b] >= 0.0 && (best < 0 || G[b] > G[best])) best = b;
    }
    *lambda = best >= 0 ? G[best] * cm->p : 0.0;
    free(v);
    return best;
}

/* ======================================================================
 * Chain verification.  [LS] Section 2.1 with the acceptance and correction
 * rules of speculative sampling (the formulas are blank in the page's text;
 * this is the Leviathan / Chen rule that [HS] Section 2 cites):
 *   accept y_i with probability min(1, p_i(y_i) / q_i(y_i))  (u_i < rho_i);
 *   at the first rejected slot sample from norm(max(0, p_i - q_i));
 *   if all b slots pass, sample the bonus from p_{b+1};
 *   the prefix advances by r + 1 tokens.
 * Point-mass slots ([HS] Section 5.8 and Appendix H) have q = delta_{y}.
 * At T = 0 the target verifies each draft as its argmax point mass
 * ([HS] Appendix H; [AS] Section 2.2): accept iff y_i = argmax, emit the
 * argmax at the first miss or after the last slot.  Argmax ties go to the
 * lowest token id.
 *
 * p_i = softmax(z_i / T), q_i = softmax(w_i / T) in fp64.  Sampling is an
 * inverse CDF with one uniform: the smallest v whose running sum (index
 * order, fp64) exceeds u' * W.  The accept test compares in fp64.
 * ====================================================================== */
typedef struct { double M; double Z; int64_t arg; int finite; } row_stats;

static row_stats stats_of(const void* base, int dtype, int64_t off, int V, double T)
{
    row_stats s;
    double mx = -INFINITY;
    int64_t am = -1;
    int finite = 1;
    for (int v = 0; v < V; ++v) {
        double z = logit_at(base, dtype, off + v);
        if (isnan(z) || z == INFINITY) finite = 0;
        if (z > mx) { mx = z; am = v; }
    }
    s.arg = am; s.finite = finite && am >= 0;
    if (T > 0.0 && s.finite) {
        double M = mx / T, Z = 0.0;
        for (int v = 0; v < V; ++v) Z += exp(logit_at(base, dtype, off + v) / T - M);
        s.M = M; s.Z = Z;
    } else { s.M = mx; s.Z = 1.0; }
    return s;
}

static double prob_of(const void* base, int dtype, int64_t off, row_stats s, double T, int64_t v)
{
    return exp(logit_at(base, dtype, off + v) / T - s.M) / s.Z;
}

/* Inverse-CDF draw over w (computed on the fly by the callback order). */
typedef struct {
    const void* tz; int tdt; int64_t toff; row_stats ts;
    const void* dz; int ddt; int64_t doff; row_stats ds;
    int mode;      /* 0: w = p ; 1: w = max(0, p - q) ; 2: w = p with w[y] = 0 */
    int64_t y;
    double T;
} resid_t;

static double resid_w(const resid_t* R, int64_t v)
{
    double p = prob_of(R->tz, R->tdt, R->toff, R->ts, R->T, v);
    if (R->mode == 0) return p;
    if (R->mode == 2) return v == R->y ? 0.0 : p;
    if (SPEC_ORACLE_MUTATION == 1) return p;
    double q = prob_of(R->dz, R->ddt, R->doff, R->ds, R->T, v);
    return p > q ? p - q : 0.0;
}

/* The draw's tie window: every token of positive weight whose CDF interval
 * [c_v, c_v + w_v) meets the band [t - eps W, t + eps W] around the target
 * t = u W.  A draw whose arithmetic differs from this one by less than eps W
 * in any running sum picks a token of the window, and no other.  Outside a
 * SAMPLE_NEAR case the window is the drawn token alone. */
static int64_t draw(const resid_t* R, int V, double u, uint32_t* flag, int64_t* win_lo, int64_t* win_hi)
{
    double W = 0.0;
    for (int64_t v = 0; v < V; ++v) W += resid_w(R, v);
    resid_t P = *R;
    if (!(W > 0.0)) {          /* unreachable in exact arithmetic */
        *flag |= OF_RESIDUAL_ZERO;
        P.mode = 0;
        W = 0.0;
        for (int64_t v = 0; v < V; ++v) W += resid_w(&P, v);
    }
    const double t = u * W, band = NEAR_EPS * W;
    double c = 0.0;
    int64_t pick = -1, lo = -1, hi = -1, lastpos = -1;
    for (int64_t v = 0; v < V; ++v) {
        double w = resid_w(&P, v);
        double c2 = c + w;
        if (w > 0.0) {
            lastpos = v;
            if (c2 > t - band && c <= t + band) {
                if (lo < 0) lo = v;
                hi = v;
            }
        }
        if (pick < 0 && c2 > t) {
            pick = v;
            if (t - c <= band || c2 - t <= band) *flag |= OF_SAMPLE_NEAR;
        }
        c = c2;
        if (pick >= 0 && c > t + band) break;   /* no later interval meets the band */
    }
    if (pick < 0) {
        *flag |= OF_SAMPLE_NEAR;   /* rounding left t at the very end: the last positive token */
        pick = lastpos >= 0 ? lastpos : V - 1;
    }
    if (lo < 0 || pick < lo) lo = pick;
    if (hi < pick) hi = pick;
    *win_lo = lo;
    *win_hi = hi;
    return pick;
}

void oracle_verify_chain(int bs, int V, double T,
                         const void* logits, int dtype, int64_t row_stride, const int64_t* row_base,
                         const void* dlogits, int ddtype, int64_t drow_stride, const int64_t* drow_base,
                         const int32_t* tokens, const uint8_t* slot_flags, int ld, const int32_t* n_slots,
                         const float* u_acc, const float* u_smp,
                         int32_t* out_tokens, int32_t* out_num, int32_t* out_accepted,
                         double* out_p, double* out_q, uint32_t* out_flags,
                         int32_t* out_win_lo, int32_t* out_win_hi)
{
    for (int r = 0; r < bs; ++r) {
        int b = n_slots[r];
        uint32_t fl = out_flags[r];
        int32_t* ot = out_tokens + (int64_t)r * (ld + 1);
        double* op = out_p + (int64_t)r * (ld + 1);
        int64_t wlo = -1, whi = -1;
        for (int i = 0; i <= ld; ++i) { ot[i] = -1; op[i] = 0.0; }
        for (int i = 0; i < ld; ++i) out_q[(int64_t)r * ld + i] = 0.0;
        int rej = -1;        /* first rejected slot, -1 if none */
        row_stats rs_rej_t, rs_rej_d;
        int64_t off_rej_t = 0, off_rej_d = 0;
        int rej_pm = 1;
        for (int i = 0; i < b; ++i) {
            int64_t toff = (row_base[r] + i) * row_stride;
            int32_t y = tokens[(int64_t)r * ld + i];
            int pm = (slot_flags[(int64_t)r * ld + i] & SLOT_POINT_MASS) != 0;
            int bad = (y < 0 || y >= V);
            if (bad) fl |= OF_BAD_TOKEN;
            row_stats ts = stats_of(logits, dtype, toff, V, T);
            if (!ts.finite) fl |= OF_BAD_LOGITS;
            double p, q = 1.0;
            row_stats qs = ts;
            int64_t doff = 0;
            if (T > 0.0) {
                p = bad ? 0.0 : prob_of(logits, dtype, toff, ts, T, y);
                if (!pm) {
                    doff = (drow_base[r] + i) * drow_stride;
                    qs = stats_of(dlogits, ddtype, doff, V, T);
                    if (!qs.finite) fl |= OF_BAD_LOGITS;
                    q = bad ? 0.0 : prob_of(dlogits, ddtype, doff, qs, T, y);
                }
            } else {
                p = (!bad && ts.arg == y) ? 1.0 : 0.0;
            }
            op[i] = p;
            out_q[(int64_t)r * ld + i] = q;
            if (rej >= 0) continue;   /* later slots: statistics only */
            int acc;
            if (T > 0.0) {
                double rho = (q > 0.0) ? p / q : 0.0;
                if (SPEC_ORACLE_MUTATION == 2) rho = p;
                double u = (double)u_acc[(int64_t)r * ld + i];
                if (fabs(u - rho) < NEAR_EPS) fl |= OF_ACCEPT_NEAR;
                acc = u < rho;
            } else {
                acc = p == 1.0;
            }
            if (acc) { ot[i] = y; continue; }
            rej = i;
            rs_rej_t = ts; off_rej_t = toff;
            rs_rej_d = qs; off_rej_d = doff;
            rej_pm = pm || bad;
        }
        int nacc = rej >= 0 ? rej : b;
        int32_t last;
        if (rej >= 0) {
            if (T > 0.0) {
                resid_t R = { logits, dtype, off_rej_t, rs_rej_t, dlogits, ddtype, off_rej_d, rs_rej_d,
                              rej_pm ? 2 : 1, tokens[(int64_t)r * ld + rej], T };
                int32_t yb = tokens[(int64_t)r * ld + rej];
                if (rej_pm && (yb < 0 || yb >= V)) R.mode = 0;
                last = (int32_t)draw(&R, V, (double)u_smp[r], &fl, &wlo, &whi);
            } else {
                last = (int32_t)rs_rej_t.arg;
            }
        } else {
            int64_t toff = (row_base[r] + b) * row_stride;
            row_stats ts = stats_of(logits, dtype, toff, V, T);
            if (!ts.finite) fl |= OF_BAD_LOGITS;
            if (T > 0.0) {
                resid_t R = { logits, dtype, toff, ts, 0, 0, 0, ts, 0, -1, T };
                last = (int32_t)draw(&R, V, (double)u_smp[r], &fl, &wlo, &whi);
                /* p of the bonus row at the bonus token */
                if (ts.finite) op[b] = prob_of(logits, dtype, toff, ts, T, last);
            } else {
                last = (int32_t)ts.arg;
                if (ts.finite) op[b] = 1.0;   /* the argmax point mass */
            }
        }
        ot[nacc] = last;
        if (wlo < 0) wlo = whi = last;   /* T = 0: the argmax, no window */
        out_win_lo[r] = (int32_t)wlo;
        out_win_hi[r] = (int32_t)whi;
        out_num[r] = nacc + 1;
        out_accepted[r] = nacc;
        out_flags[r] = fl;
    }
}

/* Commit: append the emitted tokens to each context ([LS] Section 2.1, the
 * prefix advances by r + 1).  A commit that would pass the capacity is
 * skipped and flagged. */
void oracle_commit(int bs, int32_t* ctx, int64_t ctx_stride, int32_t* ctx_len, int ctx_cap,
                   const int32_t* out_tokens, int ld1, const int32_t* out_num, uint32_t* flags)
{
    for (int r = 0; r < bs; ++r) {
        int n = out_num[r];
        if (ctx_len[r] + n > ctx_cap) { flags[r] |= OF_CTX_OVERFLOW; continue; }
        for (int i = 0; i < n; ++i) ctx[(int64_t)r * ctx_stride + ctx_len[r] + i] = out_tokens[(int64_t)r * ld1 + i];
        ctx_len[r] += n;
    }
}

/* Best-first selection of rows_cap - 1 candidates by Q (fp32 Q descending,
 * then index ascending), the S(n) curve, and the depth-first row layout
 * with children in index order ([AS] Section 3.1; Proposition 1 makes the
 * selected set parent-closed when Q does not grow along a path).  Node 0 is
 * the anchor; every parent index is below its child's. */
static void select_layout(int cnt, const int32_t* f_token, const int32_t* f_parent, const double* f_Q,
                          int rows_cap, int32_t* node_token, int32_t* parent_row, double* Q_out,
                          int32_t* n_rows, double* S_curve, uint32_t* flag)
{
    /* best-first selection of rows_cap - 1 candidates */
    int* order = (int*)malloc(sizeof(int) * (size_t)cnt);
    int m = 0;
    for (int j = 1; j < cnt; ++j) order[m++] = j;
    for (int a = 1; a < m; ++a) {           /* insertion sort: Q desc (fp32), index asc */
        int x = order[a];
        int b = a - 1;
        while (b >= 0) {
            float qb = (float)f_Q[order[b]], qx = (float)f_Q[x];
            int before = (qx > qb) || (qx == qb && x < order[b]);
            if (!before) break;
            order[b + 1] = order[b]; --b;
        }
        order[b + 1] = x;
    }
    int take = rows_cap - 1 < m ? rows_cap - 1 : m;
    for (int a = 0; a < take; ++a)
        for (int b = take; b < m; ++b) {
            double qa = f_Q[order[a]], qb = f_Q[order[b]];
            double d = fabs(qa - qb), ref = qa > qb ? qa : qb;
            if (d > 0.0 && d <= NEAR_EPS * ref) *flag |= OF_TREE_NEAR;
        }
    char* sel = (char*)calloc((size_t)cnt, 1);
    sel[0] = 1;
    for (int a = 0; a < take; ++a) sel[order[a]] = 1;
    /* S(n) for every width n: the first n - 1 nodes of the best-first order
     * ([AS] Section 3.1: a single walk down that order yields S at every
     * width) */
    if (S_curve) {
        double acc = 0.0;
        for (int n = 1; n <= rows_cap; ++n) {
            S_curve[n - 1] = acc;
            if (n - 1 < m) acc += f_Q[order[n - 1]];
        }
    }
    /* depth-first layout; an explicit stack of (node, parent row) */
    int* stack_n = (int*)malloc(sizeof(int) * (size_t)cnt);
    int* stack_p = (int*)malloc(sizeof(int) * (size_t)cnt);
    int sp = 0, row = 0;
    stack_n[sp] = 0; stack_p[sp] = -1; ++sp;
    for (int i = 0; i < rows_cap; ++i) { node_token[i] = -1; parent_row[i] = -1; Q_out[i] = 0.0; }
    while (sp > 0) {
        --sp;
        int u = stack_n[sp], pr = stack_p[sp];
        node_token[row] = (u == 0) ? -1 : f_token[u];
        parent_row[row] = pr;
        Q_out[row] = f_Q[u];
        int my = row++;
        /* push children in reverse index order so the lowest index pops first */
        for (int c = cnt - 1; c >= 1; --c)
            if (sel[c] && f_parent[c] == u) { stack_n[sp] = c; stack_p[sp] = my; ++sp; }
    }
    *n_rows = row;
    free(order); free(sel); free(stack_n); free(stack_p);
}

/* ======================================================================
 * Tree build for one request.  [AS] Section 2.2 (tree shape), Section 3.1
 * (best-first order, Proposition 1, Eq. (1)), Section 3.3 ("N-gram
 * candidates" and Eq. (6)).
 *
 * Candidate index: 0 = anchor; drafter candidate (position p = 1..P, rank
 * k = 0..Kc-1) = 1 + (p-1) Kc + k, with rank 0 the pick; the pick at p hangs
 * from the pick at p-1 (the anchor for p = 1) and its siblings from the same
 * parent.  N-gram chains from source s (0 = anchor, i = pick i) then walk
 * their draft: a step equal to an existing child of the current node marks it
 * agreed and descends; otherwise a new n-gram node is appended as a child.
 * Chains stop at depth_max below the anchor or at the end of the draft.
 * Acceptance estimate (Eq. (6) with exp(s_j) = w_j and the 'none' outcome
 * weighted by the parent's own w_none): q_j = w_j / (w_none[parent] +
 * sum of w over the parent's children).  Q_j = product of q along the path.
 * The first rows_cap-1 candidates by Q descending (ties -> lower index;
 * compared on Q rounded to fp32, the kernel's key precision) are laid out
 * depth-first from the anchor, children in index order.
 * Returns the number of forest nodes.
 * ====================================================================== */
/* ======================================================================
 * Acceptance estimates of the Eq. (6) form with its scores ([AS] Section 3.3,
 * "Form"): q_j = exp(s_j) / (1 + sum over the parent's candidates of exp(s)),
 * the 1 being the explicit none outcome (score 0), and
 *   pick:    s = a0 + a1 logit h + a2 logit sigma + psi + b_req
 *   sibling: s = a3 + a4 log r + a5 logit h + a6 logit sigma + psi + b_req
 *   n-gram:  s = logit p_src + w_bucket + psi + b_req
 * where for a drafter candidate at position p psi = psi_ctx + psi_depth[p]
 * (the context term and the depth term) and for an n-gram node psi = psi_ctx.
 * A drafter candidate that an n-gram chain also proposes (agreed) adds
 * max(0, logit p_src) + w_agreed[proposal bucket][pick or sibling]; one whose
 * parent has an n-gram proposal with another token (contradicted) subtracts
 * max(0, logit p_src) and adds w_contra[that proposal's evidence][pick or
 * sibling].  An n-gram node's evidence is the copy its chain continues, the
 * source's match length l (the feature m, or n when m = 0), or, for a token
 * of the follower fallback, its follower count l, in classes
 * e = min(7, floor(log2 l)); its bucket is 4 e + min(3, the n-gram nodes
 * above it on its path), plus 32 for a follower token (the kind).  Where
 * several proposals agree with or contradict a candidate, the one of largest
 * bucket (evidence class for a contradiction) counts.  Probabilities are
 * clamped to [1e-6, 1 - 1e-6] before their logit or log.  All in fp64.
 * ====================================================================== */
typedef struct {
    double a[7];
    double w_bucket[64];
    double w_agreed[64][2];
    double w_contra[8][2];
    double psi_depth[16];        /* by drafter position p (clamped to 15)           */
    const double* h;             /* [P] confidence head at each position             */
    const double* sigma;         /* [P] the pick's share                             */
    const double* r_share;       /* [P * Kc] a sibling's share of its siblings' total */
    double psi_ctx, b_req, p_src;
    const int32_t* ng_feat;      /* [(P + 1) * 4] (n, a, m, j) of each source's draft */
} oracle_tree_score;

static double clamp_p(double x) { return x < 1e-6 ? 1e-6 : (x > 1.0 - 1e-6 ? 1.0 - 1e-6 : x); }
static double logit_p(double x) { x = clamp_p(x); return log(x / (1.0 - x)); }

static int class_of(int l)
{
    int e = 0;
    while (e < 7 && (l >> (e + 1)) > 0) ++e;
    return e;
}

static int evidence_class(const int32_t* feat)
{
    int l = feat[2] > 0 ? feat[2] : feat[0];
    int e = 0;
    while (e < 7 && (l >> (e + 1)) > 0) ++e;
    return e;
}

int oracle_tree_build(int P, int Kc, const int32_t* block, int L, const int32_t* ng, const int32_t* ng_len,
                      const int32_t* ng_follow, const float* w_node_in, const float* w_none_in, int c_max, int depth_max, int rows_cap,
                      const oracle_tree_score* sc,
                      int32_t* node_token, int32_t* parent_row, double* Q_out, int32_t* n_rows, double* S_curve,
                      int32_t* f_token, int32_t* f_parent, int32_t* f_kind, double* f_Q, uint32_t* flag)
{
    int cnt = 1 + P * Kc;
    if (cnt > c_max) return -1;
    int* depth = (int*)calloc((size_t)c_max, sizeof(int));
    int* above = (int*)calloc((size_t)c_max, sizeof(int));      /* n-gram nodes above on the path */
    int* nbucket = (int*)malloc(sizeof(int) * (size_t)c_max);   /* n-gram node: its bucket */
    int* agree_b = (int*)malloc(sizeof(int) * (size_t)c_max);   /* drafter node: best agreeing bucket */
    for (int i = 0; i < c_max; ++i) { nbucket[i] = -1; agree_b[i] = -1; }
    f_token[0] = -1; f_parent[0] = -1; f_kind[0] = 0; depth[0] = 0;
    for (int p = 1; p <= P; ++p)
        for (int k = 0; k < Kc; ++k) {
            int idx = 1 + (p - 1) * Kc + k;
            f_token[idx] = block[(p - 1) * Kc + k];
            f_parent[idx] = (p == 1) ? 0 : 1 + (p - 2) * Kc;
            f_kind[idx] = (k == 0) ? 1 : 2;      /* 1 pick, 2 sibling */
            depth[idx] = p;
        }
    for (int s = 0; s <= P; ++s) {
        int cur = (s == 0) ? 0 : 1 + (s - 1) * Kc;
        const int e = sc ? evidence_class(sc->ng_feat + 4 * s) : 0;
        for (int t = 0; t < ng_len[s]; ++t) {
            if (depth[cur] + 1 > depth_max) break;
            int tok = ng[s * L + t];
            int found = -1;
            for (int c = 1; c < cnt; ++c)
                if (f_parent[c] == cur && f_token[c] == tok) { found = c; break; }
            const int up = above[cur] + ((f_kind[cur] & 3) == 3);   /* n-gram nodes above a child of cur */
            const int fc = ng_follow ? ng_follow[s * L + t] : 0;     /* > 0: a follower token */
            const int base = fc > 0 ? 32 + 4 * class_of(fc) : 4 * e;
            const int bucket = base + (up < 3 ? up : 3);
            if (found >= 0) {
                f_kind[found] |= 4;              /* agreed */
                if ((f_kind[found] & 3) != 3 && bucket > agree_b[found]) agree_b[found] = bucket;
                cur = found;
                continue;
            }
            if (cnt >= c_max) break;
            f_token[cnt] = tok; f_parent[cnt] = cur; f_kind[cnt] = 3; depth[cnt] = depth[cur] + 1;
            above[cnt] = up;
            nbucket[cnt] = bucket;
            cur = cnt++;
        }
    }
    /* weights: given, or exp of the Eq. (6) scores with the none outcome at 1 */
    double* wn = (double*)malloc(sizeof(double) * (size_t)cnt);
    double* wz = (double*)malloc(sizeof(double) * (size_t)cnt);
    for (int j = 0; j < cnt; ++j) {
        if (!sc) { wn[j] = (double)w_node_in[j]; wz[j] = (double)w_none_in[j]; continue; }
        wz[j] = 1.0;
        if (j == 0) { wn[j] = 0.0; continue; }
        const int kind = f_kind[j] & 3;
        double sj;
        const double lps = logit_p(sc->p_src), plus = lps > 0.0 ? lps : 0.0;
        if (kind == 3) {
            sj = lps + sc->w_bucket[nbucket[j]] + sc->psi_ctx + sc->b_req;
        } else {
            const int p = depth[j], k = (j - 1) % Kc;
            const double lh = logit_p(sc->h[p - 1]), ls = logit_p(sc->sigma[p - 1]);
            const double psi = sc->psi_ctx + sc->psi_depth[p < 15 ? p : 15];
            const int ps = kind == 1 ? 0 : 1;
            if (kind == 1) sj = sc->a[0] + sc->a[1] * lh + sc->a[2] * ls + psi + sc->b_req;
            else sj = sc->a[3] + sc->a[4] * log(clamp_p(sc->r_share[(p - 1) * Kc + k])) + sc->a[5] * lh +
                      sc->a[6] * ls + psi + sc->b_req;
            if (agree_b[j] >= 0) sj += plus + sc->w_agreed[agree_b[j]][ps];
            int contra = -1;   /* largest evidence among the parent's n-gram proposals of another token */
            for (int c = 1; c < cnt; ++c)
                if (f_parent[c] == f_parent[j] && (f_kind[c] & 3) == 3 && f_token[c] != f_token[j] &&
                    (nbucket[c] % 32) / 4 > contra)
                    contra = (nbucket[c] % 32) / 4;
            if (contra >= 0) sj += -plus + sc->w_contra[contra][ps];
        }
        wn[j] = exp(sj);
    }
    /* acceptance estimates and path products (parents precede children) */
    f_Q[0] = 1.0;
    for (int j = 1; j < cnt; ++j) {
        int par = f_parent[j];
        double den = wz[par];
        for (int c = 1; c < cnt; ++c) if (f_parent[c] == par) den += wn[c];
        f_Q[j] = f_Q[par] * (wn[j] / den);
    }
    select_layout(cnt, f_token, f_parent, f_Q, rows_cap, node_token, parent_row, Q_out, n_rows, S_curve, flag);
    free(depth);
    free(above); free(nbucket); free(agree_b); free(wn); free(wz);
    return cnt;
}

/* ======================================================================
 * Rows from a forest the caller built.  [AS] Section 3.1: the candidate
 * forest is any drafter's; a node's acceptance estimate q_j is the chance
 * it is accepted given that its parent is, so its path probability is
 * Q_j = Q_parent(j) q_j with Q = 1 at the anchor (node 0), taken in index
 * order since every parent index is below its child's.  The rows are then
 * the best-first selection and depth-first layout of the tree build.
 * n is clamped to [1, c_max] (flagged).  A node whose parent is not in
 * [0, j) or whose q is not in [0, 1] (NaN included) breaks the forest: the
 * request is flagged and its rows are the anchor alone.  Returns the number
 * of nodes used.
 * ====================================================================== */
int oracle_tree_forest(int n, int c_max, const int32_t* token, const int32_t* parent, const float* q, int rows_cap,
                       int32_t* node_token, int32_t* parent_row, double* Q_out, int32_t* n_rows, double* S_curve,
                       double* f_Q, uint32_t* flag)
{
    if (n < 1 || n > c_max) {
        *flag |= OF_BAD_LENGTH;
        n = n < 1 ? 1 : c_max;
    }
    int ok = 1;
    for (int j = 1; j < n; ++j) {
        const double qj = (double)q[j];
        if (parent[j] < 0 || parent[j] >= j || !(qj >= 0.0 && qj <= 1.0)) ok = 0;
    }
    if (!ok) {
        *flag |= OF_BAD_FOREST;
        n = 1;
    }
    f_Q[0] = 1.0;
    for (int j = 1; j < n; ++j) f_Q[j] = f_Q[parent[j]] * (double)q[j];
    select_layout(n, token, parent, f_Q, rows_cap, node_token, parent_row, Q_out, n_rows, S_curve, flag);
    return n;
}

/* ======================================================================
 * Greedy tree verification.  [AS] Section 2.2: a candidate is accepted when
 * its token equals the target's argmax at its parent's row; at most one
 * child of an accepted node can match, so the accepted nodes form a path;
 * the round commits the path and the argmax at its last node.  Argmax ties
 * go to the lowest token id.
 * ====================================================================== */
void oracle_verify_tree(int bs, int V, const void* logits, int dtype, int64_t row_stride,
                        const int64_t* row_base, const int32_t* node_token, const int32_t* parent_row,
                        const int32_t* n_rows, int rows_max,
                        int32_t* out_tokens, int32_t* out_num, int32_t* out_path_rows, int32_t* out_argmax,
                        uint32_t* out_flags)
{
    for (int r = 0; r < bs; ++r) {
        int nr = n_rows[r];
        for (int i = 0; i < rows_max; ++i) {
            out_tokens[(int64_t)r * rows_max + i] = -1;
            out_path_rows[(int64_t)r * rows_max + i] = -1;
            out_argmax[(int64_t)r * rows_max + i] = -1;
        }
        for (int i = 0; i < nr; ++i) {
            row_stats s = stats_of(logits, dtype, (row_base[r] + i) * row_stride, V, 0.0);
            if (!s.finite) out_flags[r] |= OF_BAD_LOGITS;
            out_argmax[(int64_t)r * rows_max + i] = (int32_t)s.arg;
        }
        int u = 0, n = 0;
        out_path_rows[(int64_t)r * rows_max + 0] = 0;
        for (;;) {
            int a = out_argmax[(int64_t)r * rows_max + u];
            int next = -1;
            for (int c = 1; c < nr; ++c)
                if (parent_row[(int64_t)r * rows_max + c] == u && node_token[(int64_t)r * rows_max + c] == a) {
                    next = c; break;
                }
            if (next < 0) { out_tokens[(int64_t)r * rows_max + n] = a; ++n; break; }
            out_tokens[(int64_t)r * rows_max + n] = a; ++n;
            u = next;
            out_path_rows[(int64_t)r * rows_max + n] = u;
        }
        out_num[r] = n;
    }
}
