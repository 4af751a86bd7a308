// N-gram prompt-lookup drafter (Hybrid Spark, Section 4.1 "One step" and
// Section 4.2 match features; Algorithm 1, NGRAMSCAN), with the follower
// fallback of AdaSpark's n-gram fill (Section 3.3, "N-gram candidates") on
// request: one workgroup per query, one launch (the scan itself is
// ngram_scan).
#include "ngram_scan.hpp"

namespace spec {

struct NgramParams {
    int32_t bs, nq;
    const int32_t* ctx; int64_t ctx_stride; const int32_t* ctx_len;
    const int32_t* query_req;
    const int32_t* extra; int64_t extra_stride; const int32_t* extra_len;
    int32_t n_min, n_max, max_draft, cap, follow_ctx;
    int32_t* draft; int32_t* draft_len; int32_t* feat; int32_t* follow;
};

__device__ __forceinline__ Text query_text(const NgramParams& P, int q)
{
    Text x;
    const int req = P.query_req ? P.query_req[q] : q;
    int64_t tl = 0, el = 0;
    x.a = nullptr;
    x.b = nullptr;
    if (req >= 0 && req < P.bs) {
        tl = P.ctx_len[req];
        tl = tl < 0 ? 0 : (tl > P.ctx_stride ? P.ctx_stride : tl);
        x.a = P.ctx + (int64_t)req * P.ctx_stride;
        if (P.extra && P.extra_len) {
            el = P.extra_len[q];
            el = el < 0 ? 0 : (el > P.extra_stride ? P.extra_stride : el);
            x.b = P.extra + (int64_t)q * P.extra_stride;
        }
    }
    x.na = tl;
    x.n = tl + el;
    return x;
}

// PLAIN: query q is request q and there is no extra text, so the first batch
// can be addressed before the length arrives (positions clamped into the row).
// NT threads and NB positions per thread per batch: the host picks the
// smallest window (NT * NB tokens) that holds the longest text, so a text
// takes one batch and the workgroup no more LDS than it needs.
// FOLLOW: with the follower fallback (its LDS only in these instances).
template <bool PLAIN, bool FOLLOW, int NT, int NB>
__global__ __launch_bounds__(NT) void k_ngram(NgramParams P)
{
    const int q = blockIdx.x;
    int32_t v[NB];
    if constexpr (PLAIN) {
        const int32_t* row = P.ctx + (int64_t)q * P.ctx_stride;
        const int64_t last = P.ctx_stride - 1;   // >= 0 (checked by the host)
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int64_t j = threadIdx.x + (int64_t)u * NT;
            v[u] = row[j < last ? j : last];
        }
    }
    const Text x = query_text(P, q);
    __shared__ int32_t win[NT * NB];
    __shared__ NgramShared<NT> S;
    NgramOut O;
    O.n_min = P.n_min; O.n_max = P.n_max; O.max_draft = P.max_draft; O.cap = P.cap;
    O.draft = P.draft + (int64_t)q * P.max_draft;
    O.draft_len = P.draft_len + q;
    O.feat = P.feat + 4 * (int64_t)q;
    if constexpr (FOLLOW) {
        __shared__ FollowShared FS;
        O.follow_ctx = P.follow_ctx;
        O.follow = P.follow ? P.follow + (int64_t)q * P.max_draft : nullptr;
        ngram_scan<NT, NB>(x, win, S, O, v, PLAIN, &FS);
    } else {
        O.follow_ctx = 0;
        O.follow = nullptr;
        ngram_scan<NT, NB>(x, win, S, O, v, PLAIN);
    }
}

template <bool PLAIN, bool FOLLOW>
static void launch_ngram(const NgramParams& P, int64_t text_max, hipStream_t st)
{
    if (text_max <= 512 * 10)
        hipLaunchKernelGGL((k_ngram<PLAIN, FOLLOW, 512, 10>), dim3(P.nq), dim3(512), 0, st, P);
    else if (text_max <= 512 * 16)
        hipLaunchKernelGGL((k_ngram<PLAIN, FOLLOW, 512, 16>), dim3(P.nq), dim3(512), 0, st, P);
    else if (text_max <= 1024 * 16)
        hipLaunchKernelGGL((k_ngram<PLAIN, FOLLOW, 1024, 16>), dim3(P.nq), dim3(1024), 0, st, P);
    else
        hipLaunchKernelGGL((k_ngram<PLAIN, FOLLOW, 1024, 32>), dim3(P.nq), dim3(1024), 0, st, P);
}

}  // namespace spec

using namespace spec;

size_t spec_ngram_ws(const spec_ngram_args*) { return 0; }

int spec_ngram_launch(const spec_ngram_args* a, hipStream_t st)
{
    NgramParams P;
    P.bs = a->bs; P.nq = a->nq;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len;
    P.query_req = a->query_req;
    P.extra = a->extra; P.extra_stride = a->extra ? a->extra_stride : 0; P.extra_len = a->extra_len;
    P.n_min = a->n_min; P.n_max = a->n_max; P.max_draft = a->max_draft; P.cap = a->copy_cap;
    P.follow_ctx = a->follow_ctx;
    P.draft = a->draft; P.draft_len = a->draft_len; P.feat = a->feat;
    P.follow = a->follow_ctx > 0 ? a->draft_follow : nullptr;
    const int64_t text_max = a->ctx_stride + (a->extra ? a->extra_stride : 0);
    const bool plain = !a->query_req && !a->extra && a->nq == a->bs && a->ctx_stride >= 1;
    if (a->follow_ctx > 0) {
        if (plain) launch_ngram<true, true>(P, text_max, st);
        else launch_ngram<false, true>(P, text_max, st);
    } else {
        if (plain) launch_ngram<true, false>(P, text_max, st);
        else launch_ngram<false, false>(P, text_max, st);
    }
    return spec_record_hip_error(hipGetLastError());
}
