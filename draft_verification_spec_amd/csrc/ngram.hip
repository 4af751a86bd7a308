// N-gram prompt-lookup drafter (Hybrid Spark, Section 4.1 "One step" and
// Section 4.2 match features; Algorithm 1, NGRAMSCAN).
//
// k_ngram_scan : one workgroup per (chunk of end positions, query).  The
//                query's trailing copy_cap tokens are staged in LDS; each
//                thread tests end positions j (consecutive threads read
//                consecutive tokens, so the first comparison -- where almost
//                every position stops -- is one coalesced load) and extends a
//                match backwards while tokens agree.  Matches become keys
//                (length << 32 | j), so "longest, then latest" is the largest
//                key; each workgroup keeps its top two.
// k_ngram_final: one wave per query merges the chunk top-2s, derives the
//                features (n, a, m, j) and copies the draft.
#include "common.hpp"

namespace spec {

constexpr int kScanBlock = 256;

struct NgramParams {
    int32_t bs, nq;
    const int32_t* ctx; int64_t ctx_stride; const int32_t* ctx_len;
    const int32_t* query_req;
    const int32_t* extra; int64_t extra_stride; const int32_t* extra_len;
    int32_t n_min, n_max, max_draft, cap;
    int32_t* draft; int32_t* draft_len; int32_t* feat;
    Top2* part; int32_t nsplit;
};

struct Text {
    const int32_t* a;  // context row
    int64_t na;
    const int32_t* b;  // extra row (may be null)
    int64_t n;         // total length
};

__device__ __forceinline__ Text query_text(const NgramParams& P, int q)
{
    Text x;
    int req = P.query_req ? P.query_req[q] : q;
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

__device__ __forceinline__ int32_t tok(const Text& x, int64_t p) { return p < x.na ? x.a[p] : x.b[p - x.na]; }

__global__ __launch_bounds__(kScanBlock) void k_ngram_scan(NgramParams P)
{
    const int s = blockIdx.x, q = blockIdx.y;
    const Text x = query_text(P, q);
    __shared__ int32_t suf[SPEC_MAX_CAP];
    const int64_t jlo = (int64_t)s * kNgramChunk;
    const int64_t jhi = (jlo + kNgramChunk < x.n - 1) ? jlo + kNgramChunk : x.n - 1;  // j <= n-2
    Top2 best{0, 0};
    if (jlo < jhi) {
        const int64_t ns = x.n < P.cap ? x.n : P.cap;
        for (int64_t i = threadIdx.x; i < ns; i += kScanBlock) suf[i] = tok(x, x.n - 1 - i);
        __syncthreads();
        for (int64_t j = jlo + threadIdx.x; j < jhi; j += kScanBlock) {
            const int64_t lim = (j + 1 < P.cap) ? j + 1 : P.cap;
            int64_t l = 0;
            while (l < lim && tok(x, j - l) == suf[l]) ++l;
            if (l >= P.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)j);
        }
    }
    best = wave_top2(best);
    __shared__ Top2 sh[kScanBlock / kWave];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    if (lane == 0) sh[wid] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        Top2 t = sh[0];
        for (int w = 1; w < kScanBlock / kWave; ++w) t = top2_merge(t, sh[w]);
        P.part[(int64_t)q * P.nsplit + s] = t;
    }
}

__global__ __launch_bounds__(kWave) void k_ngram_final(NgramParams P)
{
    const int q = blockIdx.x, t = threadIdx.x;
    const Text x = query_text(P, q);
    Top2 best{0, 0};
    for (int s = t; s < P.nsplit; s += kWave) best = top2_merge(best, P.part[(int64_t)q * P.nsplit + s]);
    best = wave_top2(best);
    int32_t* d = P.draft + (int64_t)q * P.max_draft;
    if (best.a == 0) {
        for (int k = t; k < P.max_draft; k += kWave) d[k] = -1;
        if (t == 0) {
            P.draft_len[q] = 0;
            P.feat[4 * (int64_t)q + 0] = 0;
            P.feat[4 * (int64_t)q + 1] = 0;
            P.feat[4 * (int64_t)q + 2] = 0;
            P.feat[4 * (int64_t)q + 3] = -1;
        }
        return;
    }
    const int64_t l = (int64_t)(best.a >> 32);
    const int64_t j = (int64_t)(best.a & 0xFFFFFFFFu);
    const int64_t avail = x.n - 1 - j;
    const int64_t len = avail < P.max_draft ? avail : P.max_draft;
    for (int k = t; k < P.max_draft; k += kWave) d[k] = (k < len) ? tok(x, j + 1 + k) : -1;
    if (t == 0) {
        int a = 1;
        if (best.b != 0) {
            const int64_t jr = (int64_t)(best.b & 0xFFFFFFFFu);
            a = tok(x, jr + 1) == tok(x, j + 1);
        }
        P.draft_len[q] = (int32_t)len;
        P.feat[4 * (int64_t)q + 0] = (int32_t)(l < P.n_max ? l : P.n_max);
        P.feat[4 * (int64_t)q + 1] = a;
        P.feat[4 * (int64_t)q + 2] = (l >= P.n_max) ? (int32_t)l : 0;
        P.feat[4 * (int64_t)q + 3] = (int32_t)j;
    }
}

}  // namespace spec

using namespace spec;

static int32_t ngram_splits(const spec_ngram_args* a)
{
    const int64_t tmax = a->ctx_stride + (a->extra ? a->extra_stride : 0);
    int64_t n = (tmax - 1 + kNgramChunk - 1) / kNgramChunk;
    return (int32_t)(n < 1 ? 1 : n);
}

size_t spec_ngram_ws(const spec_ngram_args* a) { return align256((size_t)a->nq * ngram_splits(a) * sizeof(Top2)); }

int spec_ngram_launch(const spec_ngram_args* a, hipStream_t st)
{
    NgramParams P;
    P.bs = a->bs; P.nq = a->nq;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len;
    P.query_req = a->query_req;
    P.extra = a->extra; P.extra_stride = a->extra ? a->extra_stride : 0; P.extra_len = a->extra_len;
    P.n_min = a->n_min; P.n_max = a->n_max; P.max_draft = a->max_draft; P.cap = a->copy_cap;
    P.draft = a->draft; P.draft_len = a->draft_len; P.feat = a->feat;
    P.part = (Top2*)a->workspace;
    P.nsplit = ngram_splits(a);
    hipLaunchKernelGGL(k_ngram_scan, dim3(P.nsplit, a->nq), dim3(kScanBlock), 0, st, P);
    hipLaunchKernelGGL(k_ngram_final, dim3(a->nq), dim3(kWave), 0, st, P);
    return spec_record_hip_error(hipGetLastError());
}
