// N-gram prompt-lookup drafter (Hybrid Spark, Section 4.1 "One step" and
// Section 4.2 match features; Algorithm 1, NGRAMSCAN).
//
// One workgroup of 1024 threads per query, one launch:
//   * each thread tests end positions j = t, t + 1024, ...: it loads the token
//     at j for a batch of 16 positions (independent coalesced loads, one memory
//     round trip per batch; when query q is simply request q the first batch
//     goes out before the context length is known), and the batch (16,384
//     tokens) is staged in LDS so that every later comparison reads LDS;
//   * the query's trailing copy_cap tokens are staged in LDS as well, from the
//     window when the whole text fits in it;
//   * for the rare hits a thread compares up to 4 tokens backwards itself;
//     positions still matching after 4 go to a candidate list that whole waves
//     extend 64 tokens per step with a ballot (compared up to
//     min(j + 1, copy_cap));
//   * a match of length l >= n_min becomes the key (l << 32 | j), so "longest,
//     then latest" is the largest key; the workgroup keeps the top two;
//   * thread 0 derives (n, a, m, j) and the first lanes copy the draft, from
//     the window when it holds the continuation.
#include "common.hpp"

namespace spec {

constexpr int kScanBlock = 1024;
constexpr int kBatch = 16;

struct NgramParams {
    int32_t bs, nq;
    const int32_t* ctx; int64_t ctx_stride; const int32_t* ctx_len;
    const int32_t* query_req;
    const int32_t* extra; int64_t extra_stride; const int32_t* extra_len;
    int32_t n_min, n_max, max_draft, cap;
    int32_t* draft; int32_t* draft_len; int32_t* feat;
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

// Token p of the text: the address is selected first, so a batch of these is
// a batch of independent loads rather than branches around them.
__device__ __forceinline__ int32_t tok(const Text& x, int64_t p)
{
    const uintptr_t pa = (uintptr_t)(x.a + p);
    const uintptr_t pb = (uintptr_t)x.b + (uintptr_t)((p - x.na) * (int64_t)sizeof(int32_t));
    return *(const int32_t*)(p < x.na ? pa : pb);
}

constexpr int kWin = kScanBlock * kBatch;   // tokens of one batch, staged in LDS (64 KB)
constexpr int kPre = 4;          // tokens each thread compares before handing a match to its wave
constexpr int kMaxCand = 2048;   // candidate list in LDS; overflow is extended by the thread itself

// PLAIN: query q is request q and there is no extra text, so the first batch
// can be addressed before the length arrives (positions clamped into the row).
template <bool PLAIN>
__global__ __launch_bounds__(kScanBlock) void k_ngram(NgramParams P)
{
    const int q = blockIdx.x;
    int32_t v[kBatch];
    if constexpr (PLAIN) {
        const int32_t* row = P.ctx + (int64_t)q * P.ctx_stride;
        const int64_t last = P.ctx_stride - 1;   // >= 0 (checked by the host)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t j = threadIdx.x + (int64_t)u * kScanBlock;
            v[u] = row[j < last ? j : last];
        }
    }
    const Text x = query_text(P, q);
    __shared__ int32_t suf[SPEC_MAX_CAP];
    __shared__ int32_t win[kWin];
    __shared__ Top2 sh[kScanBlock / kWave];
    __shared__ int32_t cand[kMaxCand];
    __shared__ int32_t n_cand;
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    const int64_t jend = x.n - 1;                 // end positions j < n - 1
    const int64_t ns = x.n < P.cap ? x.n : P.cap;
    // batch loads: kBatch independent loads per thread; past the text they
    // read its last position (in bounds) and are masked off later, so a
    // window holds every position of the text it covers
    auto load_batch = [&](int64_t base) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t j = base + threadIdx.x + (int64_t)u * kScanBlock;
            v[u] = tok(x, j < x.n ? j : x.n - 1);
        }
    };
    if (!PLAIN && jend > 0) load_batch(0);   // in flight while the suffix is staged
    const bool suf_in_win = x.n <= kWin;
    if (!suf_in_win)
        for (int64_t i = threadIdx.x; i < ns; i += kScanBlock) suf[i] = tok(x, x.n - 1 - i);
    if (threadIdx.x == 0) n_cand = 0;
    // token at position p < n: from the staged window when it holds p
    int64_t wbase = 0;
    auto at = [&](int64_t p) -> int32_t { return (p >= wbase && p < wbase + kWin) ? win[p - wbase] : tok(x, p); };
    Top2 best{0, 0};
    if (jend > 0) {
        // phase 1: first kPre tokens per position, thread-private
        for (int64_t base = 0; base < jend; base += kWin) {
            if (base > 0) {
                __syncthreads();   // the previous window is no longer read
                load_batch(base);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) win[threadIdx.x + u * kScanBlock] = v[u];
            wbase = base;
            __syncthreads();
            if (base == 0 && suf_in_win) {
                for (int64_t i = threadIdx.x; i < ns; i += kScanBlock) suf[i] = win[x.n - 1 - i];
                __syncthreads();
            }
            const int32_t s0 = suf[0];
            uint32_t hits = 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = base + threadIdx.x + (int64_t)u * kScanBlock;
                hits |= (uint32_t)(j < jend && v[u] == s0) << u;
            }
            while (hits) {
                const int u = __builtin_ctz(hits);
                hits &= hits - 1;
                const int64_t j = base + threadIdx.x + (int64_t)u * kScanBlock;
                const int64_t lim = (j + 1 < P.cap) ? j + 1 : P.cap;
                int64_t l = 1;
                while (l < lim && l < kPre && at(j - l) == suf[l]) ++l;
                if (l == kPre && l < lim) {
                    const int c = atomicAdd(&n_cand, 1);
                    if (c < kMaxCand) {
                        cand[c] = (int32_t)j;
                        continue;
                    }
                    while (l < lim && at(j - l) == suf[l]) ++l;   // list full: extend here
                }
                if (l >= P.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)j);
            }
        }
    }
    __syncthreads();
    // phase 2: each wave extends listed candidates 64 tokens per step
    const int nc = n_cand < kMaxCand ? n_cand : kMaxCand;
    for (int c = wid; c < nc; c += kScanBlock / kWave) {
        const int64_t j = cand[c];
        const int64_t lim = (j + 1 < P.cap) ? j + 1 : P.cap;
        int64_t l = kPre;
        for (;;) {
            const int64_t i = l + lane;
            const bool eq = i < lim && at(j - i) == suf[i];
            const uint64_t miss = ~__ballot(eq);
            if (miss == 0) {
                l += kWave;
                continue;
            }
            l += (int64_t)__builtin_ctzll(miss);
            break;
        }
        if (l > lim) l = lim;
        if (lane == 0 && l >= P.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)j);
    }
    best = wave_top2(best);
    if (lane == 0) sh[wid] = best;
    __syncthreads();
    if (wid == 0) {
        Top2 t = lane < kScanBlock / kWave ? sh[lane] : Top2{0, 0};
        t = wave_top2(t);
        int32_t* d = P.draft + (int64_t)q * P.max_draft;
        if (t.a == 0) {
            for (int k = lane; k < P.max_draft; k += kWave) d[k] = -1;
            if (lane == 0) {
                P.draft_len[q] = 0;
                P.feat[4 * (int64_t)q + 0] = 0;
                P.feat[4 * (int64_t)q + 1] = 0;
                P.feat[4 * (int64_t)q + 2] = 0;
                P.feat[4 * (int64_t)q + 3] = -1;
            }
            return;
        }
        const int64_t l = (int64_t)(t.a >> 32);
        const int64_t j = (int64_t)(t.a & 0xFFFFFFFFu);
        const int64_t avail = x.n - 1 - j;
        const int64_t len = avail < P.max_draft ? avail : P.max_draft;
        for (int k = lane; k < P.max_draft; k += kWave) d[k] = (k < len) ? at(j + 1 + k) : -1;
        if (lane == 0) {
            int a = 1;
            if (t.b != 0) {
                const int64_t jr = (int64_t)(t.b & 0xFFFFFFFFu);
                a = at(jr + 1) == at(j + 1);
            }
            P.draft_len[q] = (int32_t)len;
            P.feat[4 * (int64_t)q + 0] = (int32_t)(l < P.n_max ? l : P.n_max);
            P.feat[4 * (int64_t)q + 1] = a;
            P.feat[4 * (int64_t)q + 2] = (l >= P.n_max) ? (int32_t)l : 0;
            P.feat[4 * (int64_t)q + 3] = (int32_t)j;
        }
    }
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
    P.draft = a->draft; P.draft_len = a->draft_len; P.feat = a->feat;
    if (!a->query_req && !a->extra && a->nq == a->bs && a->ctx_stride >= 1)
        hipLaunchKernelGGL(k_ngram<true>, dim3(a->nq), dim3(kScanBlock), 0, st, P);
    else
        hipLaunchKernelGGL(k_ngram<false>, dim3(a->nq), dim3(kScanBlock), 0, st, P);
    return spec_record_hip_error(hipGetLastError());
}
