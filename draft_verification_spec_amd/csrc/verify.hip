// Chain and tree verification kernels.
//
// Chain rule: speculative sampling as on the LongSpark page ("Efficient
// speculative decoding with a fixed-cost parallel drafter", Section 2.1) --
// accept y_i with probability min(1, p_i(y_i)/q_i(y_i)); at the first reject
// draw from norm(max(0, p_i - q_i)); after the last slot draw the bonus from
// p_{b+1}.  Point-mass slots (Hybrid Spark, Section 5.8 and Appendix H) use
// q = delta_y, so their residual is p without y.  At T = 0 a draft is
// accepted iff it is the target argmax (Hybrid Spark, Appendix H; AdaSpark,
// Section 2.2).
//
// Data flow (one stream, no host synchronisation):
//   k_stats_rows : the HBM-bound pass over batches whose rows per request are
//                  near their bound: one workgroup per two adjacent 16 KB
//                  chunks of a row, on a grid (rows x chunk pairs, requests);
//                  workgroups of rows a request does not have exit at once.
//   k_plan_rows  : otherwise one workgroup lists the rows the pass reads
//   + k_stats_flat (request order: target rows, then the draft rows of
//                  probabilistic slots), and the pass takes one (row, chunk)
//                  item per workgroup from that list.
//                  Per item: an online maximum m and sum of 2^(z*c - m*c)
//                  (c = log2(e)/T; pairwise fp32 within a 32-element tile,
//                  fp64 across tiles), or at T = 0 the maximum and its first
//                  index.  (k_stats and k_stats_pipe cover rows that are not
//                  16-byte aligned and draft rows of another dtype.)
//   k_decide     : K workgroups of 512 threads per request each merge its
//                  chunk partials and find p(y), q(y) of every slot and the
//                  first rejection; workgroup 0 draws the bonus row and
//                  point-mass residuals from the chunk sums plus one chunk
//                  rescan, while a probabilistic residual max(0, p - q) is
//                  summed by all K (each streams its share of the chunks of
//                  both rows) and drawn by the last to finish.  The drawing
//                  workgroup then commits and, when asked, drafts the
//                  request's next n-gram chain from the committed context
//                  (ngram_scan).
//   k_tree_walk  : trees (T = 0): the argmax of every row, the accepted path
//                  and its commit, one wave per request.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "ngram_scan.hpp"

namespace spec {

constexpr int kBlock = 256;
constexpr int kTile = 4;              // 16-byte vectors in flight per thread per step
constexpr int kMaxLdsPrefix = 4096;   // batch sizes whose row prefix fits in LDS
constexpr int kSubSums = 16;          // residual sums per chunk (one per wave and vector slot of k_decide)

// Chunk partial: T > 0: (m, -, s); T = 0: (best, idx | bad << 31, -).
struct Partial {
    float m;
    int32_t idx;
    double s;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte vector of logits that is read once: a non-temporal load, which
// streams markedly faster than a plain load on gfx950.
__device__ __forceinline__ uint4 load_stream(const void* p)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t e)
{
    if constexpr (DT == SPEC_F32) return ((const float*)base)[e];
    else return bf16_bits_to_float(((const uint16_t*)base)[e]);
}

template <int DT>
constexpr int vec_of() { return DT == SPEC_F32 ? 4 : 8; }

template <int DT, int VEC>
__device__ __forceinline__ void loadv(const void* base, int64_t e, float* v)
{
    if constexpr (VEC == 1) {
        v[0] = load1<DT>(base, e);
    } else if constexpr (DT == SPEC_F32) {
        static_assert(VEC == 4, "fp32 vectors are 16 bytes");
        const uint4 x = load_stream((const float*)base + e);
        v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
    } else {
        static_assert(VEC == 8, "bf16 vectors are 16 bytes");
        const uint4 x = load_stream((const uint16_t*)base + e);
        v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
        v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
        v[4] = __uint_as_float(x.z << 16); v[5] = __uint_as_float(x.z & 0xFFFF0000u);
        v[6] = __uint_as_float(x.w << 16); v[7] = __uint_as_float(x.w & 0xFFFF0000u);
    }
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t stride)
{
    return (const char*)base + row * stride * (DT == SPEC_F32 ? 4 : 2);
}

__device__ __forceinline__ float logit_at(const void* base, int dt, int64_t row, int64_t stride, int64_t v)
{
    return dt == SPEC_F32 ? ((const float*)base)[row * stride + v]
                          : bf16_bits_to_float(((const uint16_t*)base)[row * stride + v]);
}

// ---------------------------------------------------------------------------
// online softmax statistics, fp64 accumulation
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ float pairwise_sum(float* t)
{
#pragma unroll
    for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w) t[i] += t[i + w];
    return t[0];
}

// Fold N values into (m, s): m = largest raw logit, s = sum of 2^(z*c - m*c).
template <int N>
__device__ __forceinline__ void sm_update(const float* v, float c, float& m, double& s)
{
    float tm = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i) tm = fmaxf(tm, v[i]);
    if (tm > m) {
        if (m != -INFINITY) s *= (double)fast_exp2((float)((double)(m * c) - (double)(tm * c)));
        m = tm;
    }
    if (m != -INFINITY) {
        const float o = m * c;
        float t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = fast_exp2(fmaf(v[i], c, -o));
        s += (double)pairwise_sum<N>(t);
    } else if (tm != tm) {
        s = __builtin_nan("");  // a tile of NaN before any finite value
    }
}

__device__ __forceinline__ void sm_combine(float& m, double& s, float m2, double s2, float c)
{
    if (m2 > m) {
        float t = m; m = m2; m2 = t;
        double u = s; s = s2; s2 = u;
    }
    if (m2 == -INFINITY) {
        if (s2 != s2) s = s2;
        return;
    }
    s += s2 * (double)fast_exp2((float)((double)(m2 * c) - (double)(m * c)));
}

struct ArgAcc {
    float best;
    int32_t idx;
    int32_t bad;
};

__device__ __forceinline__ void am_update(float v, int32_t i, ArgAcc& a)
{
    if (v > a.best) { a.best = v; a.idx = i; }
    a.bad |= (v != v) | (v == INFINITY);
}

__device__ __forceinline__ void am_combine(ArgAcc& a, const ArgAcc& b)
{
    if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) { a.best = b.best; a.idx = b.idx; }
    a.bad |= b.bad;
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& x, float* v)
{
    if constexpr (DT == SPEC_F32) {
        v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
    } else {
        v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
        v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
        v[4] = __uint_as_float(x.z << 16); v[5] = __uint_as_float(x.z & 0xFFFF0000u);
        v[6] = __uint_as_float(x.w << 16); v[7] = __uint_as_float(x.w & 0xFFFF0000u);
    }
}

// Fold kTile raw 16-byte vectors into (m, s); the sum is the pairwise tree of
// sm_update over the kTile * VEC values, unpacked one vector at a time so the
// values never all sit in registers.
template <int DT, int NV = kTile>
__device__ __forceinline__ void sm_update_raw(const uint4* raw, float c, float& m, double& s)
{
    constexpr int VEC = vec_of<DT>();
    float tm = -INFINITY;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        float v[VEC];
        unpack<DT>(raw[u], v);
#pragma unroll
        for (int q = 0; q < VEC; ++q) tm = fmaxf(tm, v[q]);
    }
    if (tm > m) {
        if (m != -INFINITY) s *= (double)fast_exp2((float)((double)(m * c) - (double)(tm * c)));
        m = tm;
    }
    if (m != -INFINITY) {
        const float o = m * c;
        float vs[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            float v[VEC];
            unpack<DT>(raw[u], v);
#pragma unroll
            for (int q = 0; q < VEC; ++q) v[q] = fast_exp2(fmaf(v[q], c, -o));
            vs[u] = pairwise_sum<VEC>(v);
        }
        s += (double)pairwise_sum<NV>(vs);
    } else if (tm != tm) {
        s = __builtin_nan("");
    }
}

template <int DT>
__device__ __forceinline__ void am_update_raw(const uint4* raw, int64_t e, ArgAcc& a)
{
    constexpr int VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
        float v[VEC];
        unpack<DT>(raw[u], v);
#pragma unroll
        for (int q = 0; q < VEC; ++q) am_update(v[q], (int32_t)(e + u * STEP + q), a);
    }
}

template <int DT>
__device__ __forceinline__ void load_raw(const void* row, int64_t e, uint4* raw)
{
    constexpr int VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    const char* b = (const char*)row + e * (DT == SPEC_F32 ? 4 : 2);
#pragma unroll
    for (int u = 0; u < kTile; ++u) raw[u] = load_stream(b + u * STEP * (DT == SPEC_F32 ? 4 : 2));
}

// Thread t of a 256-thread group folds its share of [lo, hi) (the whole
// workgroup when the group is the workgroup).
template <int DT, int VEC>
__device__ __forceinline__ void chunk_softmax(const void* row, int64_t lo, int64_t hi, float c, float& m, double& s,
                                              int t = (int)threadIdx.x)
{
    const int64_t hv = lo + (hi - lo) / VEC * VEC;
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    int64_t e = lo + (int64_t)t * VEC;
    if constexpr (VEC > 1) {
        for (; e + (kTile - 1) * STEP < hv; e += kTile * STEP) {
            uint4 raw[kTile];
            load_raw<DT>(row, e, raw);
            sm_update_raw<DT>(raw, c, m, s);
        }
    } else {
        for (; e + (kTile - 1) * STEP < hv; e += kTile * STEP) {
            float v[kTile];
#pragma unroll
            for (int u = 0; u < kTile; ++u) v[u] = load1<DT>(row, e + u * STEP);
            sm_update<kTile>(v, c, m, s);
        }
    }
    for (; e < hv; e += STEP) {
        float v[VEC];
        loadv<DT, VEC>(row, e, v);
        sm_update<VEC>(v, c, m, s);
    }
    for (int64_t x = hv + t; x < hi; x += kBlock) {
        float v = load1<DT>(row, x);
        sm_update<1>(&v, c, m, s);
    }
}

template <int DT, int VEC>
__device__ __forceinline__ void chunk_argmax(const void* row, int64_t lo, int64_t hi, ArgAcc& a,
                                             int t = (int)threadIdx.x)
{
    const int64_t hv = lo + (hi - lo) / VEC * VEC;
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    int64_t e = lo + (int64_t)t * VEC;
    if constexpr (VEC > 1) {
        for (; e + (kTile - 1) * STEP < hv; e += kTile * STEP) {
            uint4 raw[kTile];
            load_raw<DT>(row, e, raw);
            am_update_raw<DT>(raw, e, a);
        }
    } else {
        for (; e + (kTile - 1) * STEP < hv; e += kTile * STEP) {
            float v[kTile];
#pragma unroll
            for (int u = 0; u < kTile; ++u) v[u] = load1<DT>(row, e + u * STEP);
#pragma unroll
            for (int u = 0; u < kTile; ++u) am_update(v[u], (int32_t)(e + u * STEP), a);
        }
    }
    for (; e < hv; e += STEP) {
        float v[VEC];
        loadv<DT, VEC>(row, e, v);
#pragma unroll
        for (int k = 0; k < VEC; ++k) am_update(v[k], (int32_t)(e + k), a);
    }
    for (int64_t x = hv + t; x < hi; x += kBlock) am_update(load1<DT>(row, x), (int32_t)x, a);
}

__device__ __forceinline__ void bad_partial(Partial* out)
{
    if (threadIdx.x == 0) {
        Partial p;
        p.m = __builtin_nanf(""); p.idx = (int32_t)0x80000000; p.s = __builtin_nan("");
        *out = p;
    }
}

// ---------------------------------------------------------------------------
// the statistics pass
// ---------------------------------------------------------------------------

struct StatsParams {
    const void* logits; int64_t stride; const int64_t* row_base; int64_t n_rows;
    const void* dlogits; int64_t dstride; const int64_t* drow_base; int64_t dn_rows;
    const int32_t* counts;        // target rows of request r = clamp(counts[r], cmin, cmax) + cadd
    int32_t cmin, cmax, cadd;
    const uint8_t* slot_flags;    // chain: draft row k exists iff k < clamp(counts) and the slot is probabilistic
    int32_t ld;
    int32_t bs, vocab;
    int64_t chunk;
    int32_t splits;
    float c;
    Partial* part;
    int32_t NR;                   // partial rows per request
    int32_t draft_base;           // partial row of draft row k = draft_base + k
    const int32_t* gprefix;       // [bs + 1] row prefix in global memory (large batches) or null
    int2* plan;                   // flat pass: the rows it reads (k_plan_rows) ...
    int32_t* plan_count;          // ... and their count
    uint32_t* done;               // chain draws: counters k_plan_rows zeroes ([bs]) ...
    double* sums;                 // ... and residual sums it sets to -1 ([bs, splits, kSubSums]); or null
};

__device__ __forceinline__ int32_t target_rows(const StatsParams& P, int r)
{
    int c = P.counts[r];
    c = c < P.cmin ? P.cmin : (c > P.cmax ? P.cmax : c);
    return c + P.cadd;
}

// Draft rows of request r: one per probabilistic slot k < clamp(counts[r]).
__device__ __forceinline__ int32_t draft_rows(const StatsParams& P, int r)
{
    const int b = target_rows(P, r) - P.cadd;
    int32_t n = 0;
    for (int k = 0; k < b; ++k) n += !(P.slot_flags[(int64_t)r * P.ld + k] & SPEC_SLOT_POINT_MASS);
    return n;
}

// Rows the statistics pass reads for request r: its target rows, and with
// DITEMS its draft rows as well.
template <bool DITEMS>
__device__ __forceinline__ int32_t pass_rows(const StatsParams& P, int r)
{
    if constexpr (DITEMS) return target_rows(P, r) + draft_rows(P, r);
    else return target_rows(P, r);
}

// Exclusive prefix of the per-request rows over a workgroup of NT threads;
// returns the total.  With `rb` (and `drb`) the target (and draft) row bases
// are staged too, in the same round trip.
template <int NT = kBlock, bool DITEMS = false>
__device__ int32_t row_prefix(const StatsParams& P, int32_t* pre, int64_t* rb = nullptr, int64_t* drb = nullptr)
{
    __shared__ int32_t sh[NT / kWave];
    const int per = (P.bs + NT - 1) / NT;
    const int r0 = threadIdx.x * per;
    int32_t local = 0;
    for (int r = r0; r < r0 + per && r < P.bs; ++r) {
        local += pass_rows<DITEMS>(P, r);
        if (rb) rb[r] = P.row_base[r];
        if (drb) drb[r] = P.drow_base[r];
    }
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    int32_t inc = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int32_t u = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += u;
    }
    if (lane == kWave - 1) sh[wid] = inc;
    __syncthreads();
    int32_t before = 0, tot = 0;
    for (int w = 0; w < NT / kWave; ++w) {
        if (w < wid) before += sh[w];
        tot += sh[w];
    }
    int32_t run = before + inc - local;
    for (int r = r0; r < r0 + per && r < P.bs; ++r) {
        pre[r] = run;
        run += pass_rows<DITEMS>(P, r);
    }
    if (threadIdx.x == 0) pre[P.bs] = tot;
    __syncthreads();
    return tot;
}

__global__ __launch_bounds__(kBlock) void k_plan(StatsParams P, int32_t* pre)
{
    row_prefix<kBlock>(P, pre);
}

// Where one work item (verified row, chunk) lives.
struct ItemLoc {
    int r, k, s;
    int64_t row, drow;
    bool draft_row;
};

// Partials of one chunk per wave, double-buffered by item parity so that one
// barrier per item suffices.
struct BlockRed {
    float m[2][kBlock / kWave];
    double s[2][kBlock / kWave];
    int32_t i[2][kBlock / kWave];
};

// Workgroup combine of per-thread softmax state (m, s) into *out (thread 0).
__device__ __forceinline__ void block_softmax_out(float m, double s, float c, BlockRed& R, int par, Partial* out)
{
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const double s2 = __shfl_xor(s, o, kWave);
        sm_combine(m, s, m2, s2, c);
    }
    if (lane == 0) { R.m[par][wid] = m; R.s[par][wid] = s; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kBlock / kWave; ++w) sm_combine(m, s, R.m[par][w], R.s[par][w], c);
        Partial p;
        p.m = m; p.idx = 0; p.s = s;
        *out = p;
    }
}

__device__ __forceinline__ void block_argmax_out(ArgAcc acc, BlockRed& R, int par, Partial* out)
{
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        ArgAcc b{__shfl_xor(acc.best, o, kWave), __shfl_xor(acc.idx, o, kWave), __shfl_xor(acc.bad, o, kWave)};
        am_combine(acc, b);
    }
    if (lane == 0) { R.m[par][wid] = acc.best; R.i[par][wid] = acc.idx | (acc.bad ? (int32_t)0x80000000 : 0); }
    __syncthreads();
    if (threadIdx.x == 0) {
        ArgAcc t{-INFINITY, 0x7FFFFFFF, 0};
        for (int w = 0; w < kBlock / kWave; ++w) {
            ArgAcc b{R.m[par][w], R.i[par][w] & 0x7FFFFFFF, (R.i[par][w] >> 31) & 1};
            am_combine(t, b);
        }
        Partial p;
        p.m = t.best; p.idx = t.idx | (t.bad ? (int32_t)0x80000000 : 0); p.s = 0.0;
        *out = p;
    }
}

// Any chunk, read directly by the whole (256-thread) workgroup.
template <int DT, int VEC, bool GREEDY>
__device__ __forceinline__ void chunk_direct(const void* rp, int64_t lo, int64_t hi, float c, BlockRed& R, int par,
                                             Partial* out)
{
    if constexpr (GREEDY) {
        ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
        chunk_argmax<DT, VEC>(rp, lo, hi, acc);
        block_argmax_out(acc, R, par, out);
    } else {
        float m = -INFINITY;
        double s = 0.0;
        chunk_softmax<DT, VEC>(rp, lo, hi, c, m, s);
        block_softmax_out(m, s, c, R, par, out);
    }
}

constexpr int kRowBaseLds = 512;   // batches whose row bases are staged in LDS
constexpr int kRowMapLds = 4096;   // verified rows whose request is looked up in an LDS map

// The statistics pass for any layout (unaligned rows, large batches): items
// are dealt round-robin (item = block + j * grid), so the chunks the whole
// grid reads at one time form one contiguous span, and each is read directly.
template <int DT, int VEC, int DDT, int DVEC, bool GREEDY, bool DRAFT, bool GPRE>
__global__ __launch_bounds__(kBlock) void k_stats(StatsParams P)
{
    __shared__ int32_t lpre[GPRE ? 1 : kMaxLdsPrefix + 1];
    __shared__ int64_t lrb[GPRE ? 1 : kRowBaseLds];
    __shared__ int32_t lmap[GPRE ? 1 : kRowMapLds];
    __shared__ BlockRed R;
    const int32_t* pre;
    int32_t total;
    bool rb_lds = false, map_lds = false;
    if constexpr (GPRE) {
        pre = P.gprefix;
        total = pre[P.bs];
    } else {
        rb_lds = P.bs <= kRowBaseLds;
        total = row_prefix<kBlock>(P, lpre, rb_lds ? lrb : nullptr);
        pre = lpre;
        map_lds = total <= kRowMapLds;
        if (map_lds) {
            // request of every verified row
            for (int r = threadIdx.x; r < P.bs; r += blockDim.x)
                for (int q = pre[r]; q < pre[r + 1]; ++q) lmap[q] = r;
            __syncthreads();
        }
    }
    const int64_t items = (int64_t)total * P.splits;
    auto req_of = [&](int64_t rowf) -> int {
        if (map_lds) return lmap[rowf];
        int lo = 0, hi = P.bs;   // pre[lo] <= rowf < pre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (pre[mid] <= rowf) lo = mid; else hi = mid;
        }
        return lo;
    };
    int par = 0;   // flips after each reduction (each has one barrier)
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t rowf = it / P.splits;
        ItemLoc L;
        const int r = req_of(rowf);
        L.r = r;
        L.k = (int)(rowf - pre[r]);
        L.row = (rb_lds ? lrb[r] : P.row_base[r]) + L.k;
        L.s = (int)(it - rowf * P.splits);
        L.draft_row = false;
        L.drow = 0;
        if constexpr (DRAFT) {
            const int b = target_rows(P, r) - P.cadd;
            L.draft_row = L.k < b && !(P.slot_flags[(int64_t)r * P.ld + L.k] & SPEC_SLOT_POINT_MASS);
            if (L.draft_row) L.drow = P.drow_base[r] + L.k;
        }
        const int64_t clo = (int64_t)L.s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        Partial* out = P.part + ((int64_t)L.r * P.NR + L.k) * P.splits + L.s;
        if (L.row < 0 || L.row >= P.n_rows) {
            bad_partial(out);
        } else {
            chunk_direct<DT, VEC, GREEDY>(row_ptr<DT>(P.logits, L.row, P.stride), clo, chi, P.c, R, par, out);
            par ^= 1;
        }
        if constexpr (DRAFT) {
            if (L.draft_row) {
                Partial* dout = P.part + ((int64_t)L.r * P.NR + P.draft_base + L.k) * P.splits + L.s;
                if (L.drow < 0 || L.drow >= P.dn_rows) {
                    bad_partial(dout);
                } else {
                    chunk_direct<DDT, DVEC, false>(row_ptr<DDT>(P.dlogits, L.drow, P.dstride), clo, chi, P.c, R,
                                                   par, dout);
                    par ^= 1;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// the statistics pass, pipelined form
// ---------------------------------------------------------------------------
//
// Items are dealt round-robin (item = block + j * grid), so the chunks the
// whole grid reads at one time form one contiguous span and spread over every
// HBM channel.  Each thread keeps the next item's four 16-byte loads in flight
// while it reduces the current one; two register buffers alternate (the loop
// body appears twice, so no buffer is copied).  For the compiler's wait
// counts to let those loads stay in flight, every value the control flow
// depends on is wave-uniform (scalar branches), every path reads every buffer
// it loaded, and an item past the end, or of a row outside the logits, still
// goes through the (fully masked) reduction: only the final write differs.

constexpr int kGroups = 1;                 // 256-thread groups per workgroup
constexpr int kPipeBlock = kGroups * kBlock;
constexpr int kPipeMap = kRowMapLds;       // verified rows whose request the LDS map holds

struct GroupRed {
    float m[2][kGroups][kBlock / kWave];
    double s[2][kGroups][kBlock / kWave];
    int32_t i[2][kGroups][kBlock / kWave];
};

__device__ __forceinline__ Partial bad_value()
{
    Partial p;
    p.m = __builtin_nanf(""); p.idx = (int32_t)0x80000000; p.s = __builtin_nan("");
    return p;
}

// Group combine of per-thread softmax state; exactly one barrier.  Thread 0 of
// the group writes *out (the bad-row value when `bad`) unless out is null.
__device__ __forceinline__ void group_softmax_out(float m, double s, float c, GroupRed& R, int par, int g, int t,
                                                  Partial* out, bool bad)
{
    const int lane = t % kWave, w = t / kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave);
        const double s2 = __shfl_xor(s, o, kWave);
        sm_combine(m, s, m2, s2, c);
    }
    if (lane == 0) { R.m[par][g][w] = m; R.s[par][g][w] = s; }
    __syncthreads();
    if (t == 0 && out) {
        for (int w2 = 1; w2 < kBlock / kWave; ++w2) sm_combine(m, s, R.m[par][g][w2], R.s[par][g][w2], c);
        Partial p;
        p.m = m; p.idx = 0; p.s = s;
        *out = bad ? bad_value() : p;
    }
}

__device__ __forceinline__ void group_argmax_out(ArgAcc acc, GroupRed& R, int par, int g, int t, Partial* out, bool bad)
{
    const int lane = t % kWave, w = t / kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        ArgAcc b{__shfl_xor(acc.best, o, kWave), __shfl_xor(acc.idx, o, kWave), __shfl_xor(acc.bad, o, kWave)};
        am_combine(acc, b);
    }
    if (lane == 0) { R.m[par][g][w] = acc.best; R.i[par][g][w] = acc.idx | (acc.bad ? (int32_t)0x80000000 : 0); }
    __syncthreads();
    if (t == 0 && out) {
        ArgAcc a{-INFINITY, 0x7FFFFFFF, 0};
        for (int w2 = 0; w2 < kBlock / kWave; ++w2) {
            ArgAcc b{R.m[par][g][w2], R.i[par][g][w2] & 0x7FFFFFFF, (R.i[par][g][w2] >> 31) & 1};
            am_combine(a, b);
        }
        Partial p;
        p.m = a.best; p.idx = a.idx | (a.bad ? (int32_t)0x80000000 : 0); p.s = 0.0;
        *out = bad ? bad_value() : p;
    }
}

// Loads thread t's kTile vectors of [clo, chi) of a row (vector u at
// clo + t * VEC + u * kBlock * VEC); vectors at or past chi, and every vector
// when !go, load the first vector of row 0 instead (always valid, unused).
template <int DT>
__device__ __forceinline__ void group_issue(const void* logits, int64_t stride, int64_t row, bool go, int64_t clo,
                                            int64_t chi, int t, uint4* raw)
{
    constexpr int64_t VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    constexpr int ES = DT == SPEC_F32 ? 4 : 2;
    const char* rp = (const char*)row_ptr<DT>(logits, go ? row : 0, stride);
    const int64_t hi = go ? chi : 0;
    const int64_t e0 = clo + (int64_t)t * VEC;
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
        const int64_t e = e0 + u * STEP;
        raw[u] = load_stream(rp + (e < hi ? e : 0) * ES);
    }
}

// Group statistics of one chunk held in registers; vectors at or past hi read
// as -inf (they add nothing to a sum and win no argmax), and every register of
// the buffer is read on every path.
template <int DT, bool GREEDY>
__device__ __forceinline__ void group_chunk(const uint4* raw, int64_t lo, int64_t hi, float c, GroupRed& R, int par,
                                            int g, int t, Partial* out, bool bad)
{
    constexpr int64_t VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;   // -inf in every lane of a vector
    const int64_t e = lo + (int64_t)t * VEC;
    uint4 r2[kTile];
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
        const bool ok = e + u * STEP < hi;
        r2[u].x = ok ? raw[u].x : ninf; r2[u].y = ok ? raw[u].y : ninf;
        r2[u].z = ok ? raw[u].z : ninf; r2[u].w = ok ? raw[u].w : ninf;
    }
    if constexpr (GREEDY) {
        ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
        am_update_raw<DT>(r2, e, acc);
        group_argmax_out(acc, R, par, g, t, out, bad);
    } else {
        float m = -INFINITY;
        double s = 0.0;
        sm_update_raw<DT>(r2, c, m, s);
        group_softmax_out(m, s, c, R, par, g, t, out, bad);
    }
}

// Reads every register of a load buffer without using it: the loads have
// landed once it runs.  Used where the loop leaves with a prefetch that will
// never be reduced, so that the compiler's wait counts at the loop latch stay
// exact (otherwise that exit path makes every iteration wait for all loads).
__device__ __forceinline__ void drain(const uint4* raw)
{
#pragma unroll
    for (int u = 0; u < kTile; ++u) asm volatile("" : : "v"(raw[u].x), "v"(raw[u].y), "v"(raw[u].z), "v"(raw[u].w));
}

__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
}

struct PipeLoc {
    int r, prow, s;  // request, partial row, chunk
    int k;           // slot (target row k, or the draft row of slot k)
    int64_t row, drow;
    bool valid;      // a real item
    bool isd;        // a draft row taken as an item of its own
    bool row_ok;     // its row lies in the logits it reads
    bool draft_row;  // (inline drafts) the target row's slot has a probabilistic draft row
    bool drow_ok;
};

// How the pass treats draft rows: none (greedy, trees), as items of their own
// (same dtype as the target rows), or read beside each target chunk.
constexpr int kDraftNone = 0;
constexpr int kDraftItems = 1;
constexpr int kDraftInline = 2;

// Requires 16-byte aligned target rows, a vocabulary that is a multiple of one
// vector, bs <= kRowBaseLds and at most kPipeMap rows in the pass (with
// kDraftItems, target and draft rows together, and aligned draft rows of the
// target dtype).  The workgroup is kGroups groups of 256 threads; each
// iteration the groups take kGroups consecutive items.
template <int DT, int DDT, int DVEC, bool GREEDY, int DMODE>
__global__ __launch_bounds__(kPipeBlock) void k_stats_pipe(StatsParams P)
{
    constexpr bool DITEMS = DMODE == kDraftItems;
    __shared__ int32_t lpre[kRowBaseLds + 1];
    __shared__ int64_t lrb[kRowBaseLds];
    __shared__ int64_t ldrb[DITEMS ? kRowBaseLds : 1];
    __shared__ int32_t lmap[kPipeMap];   // request | partial row << 10 | draft << 20
    __shared__ GroupRed R;
    // wave-uniform, so that the loop control below is scalar
    const int32_t total =
        __builtin_amdgcn_readfirstlane(row_prefix<kPipeBlock, DITEMS>(P, lpre, lrb, DITEMS ? ldrb : nullptr));
    for (int r = threadIdx.x; r < P.bs; r += kPipeBlock) {
        int q = lpre[r];
        const int nt = target_rows(P, r);
        for (int k = 0; k < nt && q < kPipeMap; ++k) lmap[q++] = r | (k << 10);
        if constexpr (DITEMS) {
            const int b = nt - P.cadd;
            for (int k = 0; k < b && q < kPipeMap; ++k)
                if (!(P.slot_flags[(int64_t)r * P.ld + k] & SPEC_SLOT_POINT_MASS))
                    lmap[q++] = r | ((P.draft_base + k) << 10) | (1 << 20);
        }
    }
    __syncthreads();
    // at most kPipeMap rows of at most kMaxSplits chunks: 32-bit counts, so
    // that the loop control compiles to scalar compares
    const int32_t items = (total <= kPipeMap) ? total * P.splits : 0;   // host guarantees the bound
    const int32_t nsup = (items + kGroups - 1) / kGroups;
    const int32_t G = gridDim.x;
    int32_t S = blockIdx.x;
    if (S >= nsup) return;   // the whole workgroup
    const int g = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kBlock)), t = threadIdx.x % kBlock;   // g is wave-uniform
    auto locate = [&](int32_t item) -> PipeLoc {
        PipeLoc L;
        L.valid = item < items;
        const int32_t it = L.valid ? item : 0;
        const int32_t rowf = it / P.splits;
        const int32_t w = __builtin_amdgcn_readfirstlane(lmap[rowf]);
        const int r = w & 1023;
        L.r = r;
        L.prow = (w >> 10) & 1023;
        L.isd = DITEMS && ((w >> 20) & 1);
        L.k = L.isd ? L.prow - P.draft_base : L.prow;
        L.s = (int)(it - rowf * P.splits);
        if constexpr (DITEMS) {
            L.row = uniform64(L.isd ? ldrb[r] : lrb[r]) + L.k;
            L.row_ok = L.row >= 0 && L.row < (L.isd ? P.dn_rows : P.n_rows);
        } else {
            L.row = uniform64(lrb[r]) + L.k;
            L.row_ok = L.row >= 0 && L.row < P.n_rows;
        }
        L.draft_row = false;
        L.drow = 0;
        L.drow_ok = false;
        if constexpr (DMODE == kDraftInline) {
            const int b = target_rows(P, r) - P.cadd;
            L.draft_row = L.valid && L.k < b && !(P.slot_flags[(int64_t)r * P.ld + L.k] & SPEC_SLOT_POINT_MASS);
            if (L.draft_row) L.drow = P.drow_base[r] + L.k;
            L.drow_ok = L.drow >= 0 && L.drow < P.dn_rows;
        }
        return L;
    };
    auto issue = [&](const PipeLoc& L, uint4* raw) {
        const int64_t clo = (int64_t)L.s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        const void* base = P.logits;
        int64_t stride = P.stride;
        if constexpr (DITEMS) {
            base = L.isd ? P.dlogits : P.logits;
            stride = L.isd ? P.dstride : P.stride;
        }
        group_issue<DT>(base, stride, L.row, L.valid && L.row_ok, clo, chi, t, raw);
    };
    int par = 0;
    auto reduce = [&](const PipeLoc& L, const uint4* raw) {
        const int64_t clo = (int64_t)L.s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        Partial* out = L.valid ? P.part + ((int64_t)L.r * P.NR + L.prow) * P.splits + L.s : nullptr;
        group_chunk<DT, GREEDY>(raw, clo, (L.valid && L.row_ok) ? chi : clo, P.c, R, par, g, t, out, !L.row_ok);
        par ^= 1;
        if constexpr (DMODE == kDraftInline) {
            // every group takes this barrier too, with an empty range when it has no draft row
            const bool go = L.draft_row && L.drow_ok;
            Partial* dout = L.draft_row ? P.part + ((int64_t)L.r * P.NR + P.draft_base + L.k) * P.splits + L.s : nullptr;
            float m = -INFINITY;
            double s = 0.0;
            chunk_softmax<DDT, DVEC>(row_ptr<DDT>(P.dlogits, go ? L.drow : 0, P.dstride), clo, go ? chi : clo, P.c,
                                     m, s, t);
            group_softmax_out(m, s, P.c, R, par, g, t, dout, !L.drow_ok);
            par ^= 1;
        }
    };
    // One exit, at the latch, and both paths into it have read `rb`: the
    // compiler's wait counts at the loop header then cover only the loads of
    // the item about to be reduced.
    uint4 ra[kTile], rb[kTile];
    PipeLoc la = locate(S * kGroups + g), lb = la;
    issue(la, ra);
    bool more;
    do {
        const int32_t S1 = S + G;
        const bool m1 = S1 < nsup;   // uniform over the workgroup
        lb = locate(m1 ? S1 * kGroups + g : items);
        issue(lb, rb);
        reduce(la, ra);
        bool m2 = false;
        if (m1) {
            const int32_t S2 = S1 + G;
            m2 = S2 < nsup;
            la = locate(m2 ? S2 * kGroups + g : items);
            issue(la, ra);
            reduce(lb, rb);
            S = S2;
        } else {
            drain(rb);
        }
        more = m1 && m2;
    } while (more);
    drain(ra);
}

// ---------------------------------------------------------------------------
// the statistics pass, flat form
// ---------------------------------------------------------------------------
//
// One (row, chunk) item per workgroup, items in row-major order over a row
// list that one small workgroup writes first.  The hardware dispatcher hands
// a compute unit its next workgroup as soon as one retires, which balances
// the load better than any static deal of items over resident workgroups,
// and each item costs a single scalar load of its plan entry before its
// chunk loads go out.  The grid is sized by the host from a bound of the rows
// (surplus workgroups exit at once; a short grid strides over the rest).

// The rows of the pass in request order -- target rows 0..n-1, then with
// DITEMS the draft rows of the probabilistic slots -- as (row in its logits
// buffer or -1 outside it, partial row r * NR + prow with bit 31 set for a
// draft row); then their count.  One workgroup.
template <bool DITEMS>
__global__ __launch_bounds__(kBlock) void k_plan_rows(StatsParams P)
{
    __shared__ int32_t wsum[kBlock / kWave];
    const int t = threadIdx.x, lane = t % kWave, wid = t / kWave;
    int32_t carry = 0;
    for (int r0 = 0; r0 < P.bs; r0 += kBlock) {
        const int r = r0 + t;
        int32_t nt = 0;
        uint32_t prob = 0;   // probabilistic slots among the first b (b <= 32)
        int64_t tb = 0, db = 0;
        if (r < P.bs) {
            nt = target_rows(P, r);
            tb = P.row_base[r];
            if constexpr (DITEMS) {
                db = P.drow_base[r];
                // every flag load of the request in flight at once, beside the
                // count's (the bound is ld, not the count)
                const uint8_t* fl = P.slot_flags + (int64_t)r * P.ld;
#pragma unroll
                for (int k = 0; k < SPEC_MAX_DRAFT; ++k)
                    if (k < P.ld) prob |= (uint32_t)!(fl[k] & SPEC_SLOT_POINT_MASS) << k;
                const int b = nt - P.cadd;   // slots k < b only
                prob &= b >= 32 ? ~0u : ((1u << b) - 1u);
            }
        }
        const int32_t n = nt + (int32_t)__popc(prob);
        const int32_t inc = (int32_t)wave_incl_add((uint32_t)n);
        if (lane == kWave - 1) wsum[wid] = inc;
        __syncthreads();
        int32_t q = carry + inc - n, tile = 0;
        for (int w = 0; w < kBlock / kWave; ++w) {
            if (w < wid) q += wsum[w];
            tile += wsum[w];
        }
        if (r < P.bs) {
            for (int k = 0; k < nt; ++k) {
                const int64_t row = tb + k;
                P.plan[q++] = make_int2(row >= 0 && row < P.n_rows ? (int32_t)row : -1, r * P.NR + k);
            }
            if constexpr (DITEMS) {
                for (uint32_t m = prob; m; m &= m - 1) {
                    const int k = __builtin_ctz(m);
                    const int64_t row = db + k;
                    P.plan[q++] = make_int2(row >= 0 && row < P.dn_rows ? (int32_t)row : -1,
                                            (r * P.NR + P.draft_base + k) | (int32_t)0x80000000);
                }
            }
        }
        carry += tile;
        __syncthreads();   // wsum is rewritten by the next tile
    }
    if (t == 0) *P.plan_count = carry;
    if (P.done) {
        for (int r = t; r < 2 * P.bs; r += kBlock) P.done[r] = 0;   // counts, then chunk counters
        for (int64_t i = t; i < (int64_t)P.bs * P.splits * kSubSums; i += kBlock) P.sums[i] = -1.0;
    }
}

// Requires 16-byte aligned rows, a vocabulary that is a multiple of one
// vector and (with DITEMS) draft rows of the target dtype, also aligned.
template <int DT, bool GREEDY, bool DITEMS>
__global__ __launch_bounds__(kBlock) void k_stats_flat(StatsParams P)
{
    __shared__ GroupRed R;
    const int t = threadIdx.x;
    // the host sizes the plan for every row the pass can have, so the first
    // entry is read before the count is known (both loads in one round trip)
    const uint32_t splits = (uint32_t)P.splits;
    uint32_t it = blockIdx.x;   // < 2^31, and so is the grid: it + grid does not wrap
    int2 e = P.plan[it / splits];
    const uint32_t items = (uint32_t)__builtin_amdgcn_readfirstlane(*P.plan_count) * splits;
    int par = 0;
    while (it < items) {
        const uint32_t q = it / splits;
        const int32_t s = (int32_t)(it - q * splits);
        const int32_t row = __builtin_amdgcn_readfirstlane(e.x);
        const int32_t pr = __builtin_amdgcn_readfirstlane(e.y);
        const bool isd = DITEMS && pr < 0;
        const void* base = isd ? P.dlogits : P.logits;
        const int64_t stride = isd ? P.dstride : P.stride;
        const bool ok = row >= 0;
        const int64_t clo = (int64_t)s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        uint4 raw[kTile];
        group_issue<DT>(base, stride, row, ok, clo, chi, t, raw);
        Partial* out = P.part + (int64_t)(pr & 0x7FFFFFFF) * P.splits + s;
        group_chunk<DT, GREEDY>(raw, clo, ok ? chi : clo, P.c, R, par, 0, t, out, !ok);
        par ^= 1;
        it += gridDim.x;
        if (it < items) e = P.plan[it / splits];
    }
}

// (m, s) of a wave with DPP, valid in lane 63: the wave's largest m first
// (an inclusive max scan over rows of 16 lanes, then across rows), then each
// lane's s rescaled to it and the sum taken in fp64.  A lane with m = -inf
// adds nothing (or its NaN); the order of the fp64 additions is fixed.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v)
{
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, ROWS, 0xf, false);
    return fmaxf(v, __int_as_float(o));
}

__device__ __forceinline__ void wave_softmax_dpp(float& m, double& s, float c)
{
    float M = m;
    M = dpp_max_step<0x111, 0xf>(M);   // row_shr:1
    M = dpp_max_step<0x112, 0xf>(M);   // row_shr:2
    M = dpp_max_step<0x114, 0xf>(M);   // row_shr:4
    M = dpp_max_step<0x118, 0xf>(M);   // row_shr:8
    M = dpp_max_step<0x142, 0xa>(M);   // row_bcast:15
    M = dpp_max_step<0x143, 0xc>(M);   // row_bcast:31
    M = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), 63));
    double sc;
    if (m == -INFINITY) sc = (s != s) ? s : 0.0;
    else sc = s * (double)fast_exp2((float)((double)(m * c) - (double)(M * c)));
    s = wave_total_f64(sc);
    m = M;
}

// A workgroup of 256 threads reduces two chunks at once: threads 0..127 take
// the first, 128..255 the second, each thread NV = 2 kTile 16-byte vectors of
// its chunk (vector u at lo + tt * VEC + u * 128 * VEC, tt = t mod 128), so
// every wave reduces once per pair.  Vectors at or past hi (and every vector
// when !go) load the first vector of row 0 instead and read as -inf.
constexpr int kHalf = kBlock / 2;
constexpr int kHalfVecs = 2 * kTile;

template <int DT>
__device__ __forceinline__ void half_issue(const void* logits, int64_t stride, int64_t row, bool go, int64_t lo,
                                           int64_t hi, int tt, uint4* raw)
{
    constexpr int64_t VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kHalf * VEC;
    constexpr int ES = DT == SPEC_F32 ? 4 : 2;
    const char* rp = (const char*)row_ptr<DT>(logits, go ? row : 0, stride);
    const int64_t h = go ? hi : 0;
    const int64_t e0 = lo + (int64_t)tt * VEC;
#pragma unroll
    for (int u = 0; u < kHalfVecs; ++u) {
        const int64_t e = e0 + u * STEP;
        raw[u] = load_stream(rp + (e < h ? e : 0) * ES);
    }
}

struct HalfRed {
    float m[2][kBlock / kWave];   // by item parity, so one barrier per item suffices
    double s[2][kBlock / kWave];
};

// Softmax statistics of the half's chunk [lo, hi) from its registers; thread
// tt = 0 of the half writes *out (the bad-row value when `bad`) unless out is
// null.  One barrier, taken by the whole workgroup.
template <int DT>
__device__ __forceinline__ void half_softmax(const uint4* raw, int64_t lo, int64_t hi, float c, HalfRed& R, int par,
                                             int t, Partial* out, bool bad)
{
    constexpr int64_t VEC = vec_of<DT>();
    constexpr int64_t STEP = (int64_t)kHalf * VEC;
    const uint32_t ninf = DT == SPEC_F32 ? 0xFF800000u : 0xFF80FF80u;   // -inf in every lane of a vector
    const int tt = t % kHalf;
    const int64_t e = lo + (int64_t)tt * VEC;
    float m = -INFINITY;
    double s = 0.0;
    if (lo + STEP * kHalfVecs <= hi) {
        // a whole chunk (every chunk of a row but its last): no masking
        sm_update_raw<DT, kHalfVecs>(raw, c, m, s);
    } else {
        uint4 r2[kHalfVecs];
#pragma unroll
        for (int u = 0; u < kHalfVecs; ++u) {
            const bool ok = e + u * STEP < hi;
            r2[u].x = ok ? raw[u].x : ninf; r2[u].y = ok ? raw[u].y : ninf;
            r2[u].z = ok ? raw[u].z : ninf; r2[u].w = ok ? raw[u].w : ninf;
        }
        sm_update_raw<DT, kHalfVecs>(r2, c, m, s);
    }
    wave_softmax_dpp(m, s, c);
    const int lane = t % kWave, w = t / kWave;
    if (lane == kWave - 1) { R.m[par][w] = m; R.s[par][w] = s; }
    __syncthreads();
    if (tt == 0 && out) {
        // the half's two waves (each wave's total sits in its lane 63)
        m = R.m[par][w];
        s = R.s[par][w];
        sm_combine(m, s, R.m[par][w + 1], R.s[par][w + 1], c);
        Partial p;
        p.m = m; p.idx = 0; p.s = s;
        *out = bad ? bad_value() : p;
    }
}

// The flat pass at T > 0 with workgroups of 128 threads (two waves), one item
// each, eight 16-byte vectors per thread: each wave reduces once per chunk.
template <int DT, bool DITEMS>
__global__ __launch_bounds__(kHalf) void k_stats_flat_half(StatsParams P)
{
    __shared__ HalfRed HR;
    const int t = threadIdx.x;
    const uint32_t splits = (uint32_t)P.splits;
    uint32_t it = blockIdx.x;   // < 2^31, and so is the grid: it + grid does not wrap
    int2 e = P.plan[it / splits];
    const uint32_t items = (uint32_t)__builtin_amdgcn_readfirstlane(*P.plan_count) * splits;
    int par = 0;
    while (it < items) {
        const uint32_t q = it / splits;
        const int32_t s = (int32_t)(it - q * splits);
        const int32_t row = __builtin_amdgcn_readfirstlane(e.x);
        const int32_t pr = __builtin_amdgcn_readfirstlane(e.y);
        const bool isd = DITEMS && pr < 0;
        const void* base = isd ? P.dlogits : P.logits;
        const int64_t stride = isd ? P.dstride : P.stride;
        const bool ok = row >= 0;
        const int64_t clo = (int64_t)s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        uint4 raw[kHalfVecs];
        half_issue<DT>(base, stride, row, ok, clo, chi, t, raw);
        Partial* out = P.part + (int64_t)(pr & 0x7FFFFFFF) * P.splits + s;
        half_softmax<DT>(raw, clo, ok ? chi : clo, P.c, HR, par, t, out, !ok);
        par ^= 1;
        it += gridDim.x;
        if (it < items) e = P.plan[it / splits];
    }
}

// The same pass without a row list, for batches whose rows per request are
// close to their bound: grid ((TM + DM) * pairs, bs) with TM the target rows
// and DM the draft slots a request can have and pairs = ceil(splits / 2);
// workgroup (x, r) takes chunks 2 (x % pairs) and the next one of request
// r's target row j = x / pairs (j < TM) or of the draft row of slot j - TM,
// and exits when the request has no such row.  Both chunks' loads go out
// first, so the second chunk's data arrives while the first is reduced (a
// workgroup holds 32 KB in flight; 2% faster than one chunk each).  Its
// inputs are a handful of uniform words, read with scalar loads in one round
// trip (the slot's flag byte through its aligned word).  Workgroup (0, r) also
// resets request r's residual bookkeeping.
template <int DT, bool GREEDY, bool DITEMS>
__global__ __launch_bounds__(kBlock) void k_stats_rows(StatsParams P, int32_t TM)
{
    __shared__ GroupRed R;
    __shared__ HalfRed HR;
    const int t = threadIdx.x;
    const int r = blockIdx.y;
    const int32_t npair = (P.splits + 1) / 2;
    const int32_t j = (int32_t)blockIdx.x / npair;
    const int32_t s = 2 * ((int32_t)blockIdx.x - j * npair);   // the first of the two chunks
    const int k = j - TM;   // the draft slot, when j >= TM
    // every input first, before any store (so that they stay scalar loads)
    const int32_t nt = target_rows(P, r);
    const int64_t tb = P.row_base[r];
    int64_t db = 0;
    uint32_t f = 0;
    if constexpr (DITEMS) {
        db = P.drow_base[r];
        const int64_t off = (int64_t)r * P.ld + (k < 0 ? 0 : k);
        f = *(const uint32_t*)(P.slot_flags + (off & ~(int64_t)3)) >> (8 * (off & 3));   // via the aligned word
    }
    // all of them in one round trip: without this the compiler sinks each
    // load into the branch that uses it, one dependent trip after another
    asm volatile("" : : "s"(nt), "s"(tb), "s"(db), "s"(f));
    int64_t row;
    int32_t prow;
    bool isd = false;
    bool live;
    if (j < TM) {
        live = j < nt;
        row = tb + j;
        prow = j;
    } else {
        live = DITEMS && k < nt - P.cadd && !(f & SPEC_SLOT_POINT_MASS);
        row = db + k;
        prow = P.draft_base + k;
        isd = true;
    }
    if (live) {
        const bool ok = row >= 0 && row < (isd ? P.dn_rows : P.n_rows);
        const void* base = isd ? P.dlogits : P.logits;
        const int64_t stride = isd ? P.dstride : P.stride;
        const int64_t clo = (int64_t)s * P.chunk;
        const int64_t chi = (clo + P.chunk < P.vocab) ? clo + P.chunk : P.vocab;
        const bool two = s + 1 < P.splits;   // an odd last pair has one chunk
        const int64_t clo1 = clo + P.chunk;
        const int64_t chi1 = two ? ((clo1 + P.chunk < P.vocab) ? clo1 + P.chunk : P.vocab) : clo1;
        Partial* out = P.part + ((int64_t)r * P.NR + prow) * P.splits + s;
        if constexpr (GREEDY) {
            uint4 raw[kTile], raw1[kTile];
            group_issue<DT>(base, stride, row, ok, clo, chi, t, raw);
            group_issue<DT>(base, stride, row, ok && two, clo1, chi1, t, raw1);
            group_chunk<DT, GREEDY>(raw, clo, ok ? chi : clo, P.c, R, 0, 0, t, out, !ok);
            group_chunk<DT, GREEDY>(raw1, clo1, (ok && two) ? chi1 : clo1, P.c, R, 1, 0, t, two ? out + 1 : nullptr,
                                    !ok);
        } else {
            // each half of the workgroup reduces one chunk of the pair
            const bool second = t >= kHalf;
            const int64_t lo = second ? clo1 : clo;
            const int64_t hi = second ? ((ok && two) ? chi1 : clo1) : (ok ? chi : clo);
            uint4 raw[kHalfVecs];
            half_issue<DT>(base, stride, row, second ? (ok && two) : ok, lo, hi, t % kHalf, raw);
            half_softmax<DT>(raw, lo, hi, P.c, HR, 0, t, second ? (two ? out + 1 : nullptr) : out, !ok);
        }
    }
    if (P.done && blockIdx.x == 0) {
        if (t == 0) { P.done[r] = 0; P.done[P.bs + r] = 0; }   // count, chunk counter
        for (int i = t; i < P.splits * kSubSums; i += kBlock) P.sums[(int64_t)r * P.splits * kSubSums + i] = -1.0;
    }
}

// ---------------------------------------------------------------------------
// merging partials
// ---------------------------------------------------------------------------

// Argmax of a row from its chunk partials p[0], p[st], ... (first index on ties).
__device__ __forceinline__ bool merge_argmax(const Partial* p, int splits, int st, int32_t* idx)
{
    ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
    for (int s = 0; s < splits; ++s) {
        const Partial q = p[s * st];
        ArgAcc b{q.m, q.idx & 0x7FFFFFFF, (q.idx >> 31) & 1};
        if (q.m != q.m) b.bad = 1;
        am_combine(acc, b);
    }
    *idx = acc.idx;
    return !acc.bad && acc.idx != 0x7FFFFFFF;
}

// ---------------------------------------------------------------------------
// drawing a token by inverse CDF
// ---------------------------------------------------------------------------

struct ChainParams {
    int32_t bs, vocab, ld;
    float c;            // log2(e) / T (T > 0)
    int32_t greedy;
    const void* logits; int32_t dt; int64_t stride; const int64_t* row_base; int64_t n_rows;
    const void* dlogits; int32_t ddt; int64_t dstride; const int64_t* drow_base; int64_t dn_rows;
    const int32_t* tokens; const uint8_t* slot_flags; const int32_t* n_slots;
    const float* u_acc; const float* u_smp;
    int32_t rng; uint64_t rng_seed, rng_offset;   // uniforms drawn here (Philox4x32-10) instead of read
    int32_t* accept_hist;       // optional [ld + 1]: += 1 at the request's accepted count
    int32_t* out_tokens; int32_t* out_num; int32_t* out_acc; float* out_p; float* out_q; uint32_t* out_flags;
    int32_t write_flags;        // out_flags written (by the drawing workgroup) rather than OR-ed
    int32_t* ctx; int64_t ctx_stride; const int32_t* ctx_len; int32_t* ctx_len_out; int32_t ctx_cap;
    int32_t* ng_draft; int32_t* ng_len; int32_t* ng_feat;   // next n-gram draft after the commit, or null
    int32_t ng_min, ng_max, ng_ld, ng_cap;
    Partial* part; int32_t NR; int32_t splits; int64_t chunk;
    double* sums;               // [bs, splits, kSubSums] residual sums (-1 until written)
    uint32_t* done;             // [bs] workgroups of a request done with their residual chunks
    int32_t wait_limit;         // polls of a published residual sum before the drawer sums it itself (< 0: none)
    bool t_aligned, d_aligned;  // rows allow 16-byte vector loads
    bool coal;                  // same dtype, aligned rows, vocab a multiple of a vector
};

// Weight of token v: mode 1 = 2^(z*c - Ot) ; 3 = the same with y removed ; 2 = max(0, ep - eq * Zt/Zd).
struct Draw {
    int32_t mode;
    int32_t y;
    float Ot, Od;
    int64_t row_t, row_d;
    double ratio;
};

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11): ten rounds of two 32x32 -> 64-bit products of
// counter words 0 and 2 with the rounds' multipliers, the high halves mixed
// with the other two words and the key, the key bumped by the Weyl constants.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint2 k)
{
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
        k.x += 0x9E3779B9u;   // the bump after the last round is unused
        k.y += 0xBB67AE85u;
    }
    return c;
}

// Uniform k of request r at step `offset`: word k mod 4 of block
// Philox4x32-10(counter (k / 4, r, offset), key seed), as (w >> 8) 2^-24.
// u_accept[r][i] is uniform i and u_sample[r] uniform SPEC_MAX_DRAFT.
__device__ __forceinline__ float step_uniform(const ChainParams& P, int r, int k)
{
    const uint4 w = philox4x32_10(make_uint4((uint32_t)(k / 4), (uint32_t)r, (uint32_t)P.rng_offset,
                                             (uint32_t)(P.rng_offset >> 32)),
                                  make_uint2((uint32_t)P.rng_seed, (uint32_t)(P.rng_seed >> 32)));
    const int q = k % 4;
    const uint32_t x = q == 0 ? w.x : (q == 1 ? w.y : (q == 2 ? w.z : w.w));
    return (float)(x >> 8) * (1.0f / 16777216.0f);
}

// A decide workgroup is kDBlock threads.
constexpr int kDBlock = 512;
constexpr int kDWaves = kDBlock / kWave;

__device__ double block_sum_f64(double v)
{
    __shared__ double sh[kDWaves];
    v = wave_incl_f64(v);   // the wave's total in lane 63
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    __syncthreads();
    if (lane == kWave - 1) sh[wid] = v;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < kDWaves; ++w) tot += sh[w];
    return tot;
}

// Each thread owns a contiguous segment of up to kSeg entries of a chunk and
// loads it with 16-byte vectors when the rows allow (chunks are <= 8192
// entries, so kDBlock threads x kSeg entries cover one).
constexpr int kSeg = 16;
static_assert(kDBlock * kSeg * 2 == kChunkBytes, "a decide workgroup covers one bf16 chunk");

template <int DT>
__device__ __forceinline__ void load_seg(const void* row, bool aligned, int64_t a, int64_t b, float* v)
{
    if (aligned && b - a == kSeg) {
        constexpr int VEC = vec_of<DT>();
#pragma unroll
        for (int u = 0; u < kSeg / VEC; ++u) loadv<DT, VEC>(row, a + u * VEC, v + u * VEC);
    } else {
#pragma unroll
        for (int u = 0; u < kSeg; ++u) v[u] = (a + u < b) ? load1<DT>(row, a + u) : -INFINITY;
    }
}

// Logits of the segment [a, b) of the draw's row(s): z of the target row and,
// for a residual draw, x of the draft row (else zeros).
template <int DTT, int DTD>
__device__ __forceinline__ void seg_load(const ChainParams& P, const Draw& d, int64_t a, int64_t b, float* z, float* x)
{
    load_seg<DTT>(row_ptr<DTT>(P.logits, d.row_t, P.stride), P.t_aligned, a, b, z);
    if (d.mode == 2) {
        load_seg<DTD>(row_ptr<DTD>(P.dlogits, d.row_d, P.dstride), P.d_aligned, a, b, x);
    } else {
#pragma unroll
        for (int u = 0; u < kSeg; ++u) x[u] = 0.0f;
    }
}

// Weight of entry a + u of a segment [a, b) from its logits: mode 1 p's
// weight, 3 the same with y removed, 2 the residual max(0, ep - eq Zt/Zd).
__device__ __forceinline__ double seg_w(const ChainParams& P, const Draw& d, int64_t a, int64_t b, int u, float z,
                                        float x)
{
    const double ep = (double)fast_exp2(fmaf(z, P.c, -d.Ot));
    if (d.mode == 2) {
        const double eq = (double)fast_exp2(fmaf(x, P.c, -d.Od));
        const double v = ep - eq * d.ratio;
        return (a + u < b && v > 0.0) ? v : 0.0;
    }
    return (a + u < b && !(d.mode == 3 && a + u == d.y)) ? ep : 0.0;
}

__device__ __forceinline__ void seg_of(int64_t lo, int64_t hi, int64_t* a, int64_t* b)
{
    int64_t x = lo + (int64_t)threadIdx.x * kSeg;
    int64_t y = x + kSeg;
    *a = x < hi ? x : hi;
    *b = y < hi ? y : hi;
}

// Sum of the weights over one chunk [lo, hi) (fp64, workgroup-wide).
template <int DTT, int DTD>
__device__ double range_sum(const ChainParams& P, const Draw& d, int64_t lo, int64_t hi)
{
    int64_t a, b;
    seg_of(lo, hi, &a, &b);
    double acc = 0.0;
    if (a < b) {
        float z[kSeg], x[kSeg];
        seg_load<DTT, DTD>(P, d, a, b, z, x);
#pragma unroll
        for (int u = 0; u < kSeg; ++u) acc += seg_w(P, d, a, b, u, z[u], x[u]);
    }
    return block_sum_f64(acc);
}

// First token of the chunk [lo, hi) whose running weight (index order)
// exceeds t; when rounding leaves t past the chunk, its last positive-weight
// token; -1 if the chunk has no weight.  Each thread keeps the running sums
// of its own segment (fp64) from the one pass over its logits; the
// segments' offsets come from a DPP scan in each wave and the waves' totals
// in LDS.  A thread then marks the entries of positive weight whose running
// sum passes t; the first thread with a mark holds the token (a segment past
// the crossing marks only entries after it, and the minimum discards them).
template <int DTT, int DTD>
__device__ int64_t search_range(const ChainParams& P, const Draw& d, int64_t lo, int64_t hi, double t)
{
    __shared__ double sh_w[kDWaves];          // each wave's total
    __shared__ long long sh_found[kDWaves];   // each wave's first candidate
    __shared__ long long sh_lp[kDWaves];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    int64_t a, b;
    seg_of(lo, hi, &a, &b);
    double run[kSeg];
    double mine = 0.0;
    uint32_t posmask = 0;   // segment offsets with positive weight
    {
        float z[kSeg], x[kSeg];
        if (a < b) seg_load<DTT, DTD>(P, d, a, b, z, x);
#pragma unroll
        for (int u = 0; u < kSeg; ++u) {
            const double w = a < b ? seg_w(P, d, a, b, u, z[u], x[u]) : 0.0;
            mine += w;
            run[u] = mine;
            posmask |= (w > 0.0 ? 1u : 0u) << u;
        }
    }
    const double inc = wave_incl_f64(mine);
    if (lane == kWave - 1) sh_w[wid] = inc;
    __syncthreads();
    double cum = inc - mine;
    for (int w2 = 0; w2 < kDWaves; ++w2)
        if (w2 < wid) cum += sh_w[w2];
    uint32_t hit = 0;
#pragma unroll
    for (int u = 0; u < kSeg; ++u) hit |= (uint32_t)(cum + run[u] > t) << u;
    hit &= posmask;
    // candidates are ordered like their positions, so a wave's first
    // candidate lane holds its smallest position
    // (read across lanes with the whole wave active: under `lane == 0` the
    // compiler may compute pos for lane 0 alone)
    const uint64_t cand = __ballot(hit != 0u);
    const long long pos = a + (hit ? __builtin_ctz(hit) : 0);
    const int fl = cand ? (int)__builtin_ctzll(cand) : 0;
    const long long first = ((long long)__builtin_amdgcn_readlane((int)(pos >> 32), fl) << 32) |
                            (unsigned)__builtin_amdgcn_readlane((int)pos, fl);
    if (lane == 0) sh_found[wid] = cand ? first : -1;
    __syncthreads();
    int64_t res = -1;
    for (int w2 = 0; w2 < kDWaves; ++w2)
        if (sh_found[w2] >= 0 && (res < 0 || sh_found[w2] < res)) res = sh_found[w2];
    if (res < 0) {
        // rounding left t past the chunk: its last positive-weight token
        const long long lp = posmask ? (long long)(a + 31 - __builtin_clz(posmask)) : -1ll;
        const long long m = wave_max(lp);
        if (lane == 0) sh_lp[wid] = m;
        __syncthreads();
        for (int w2 = 0; w2 < kDWaves; ++w2) res = sh_lp[w2] > res ? sh_lp[w2] : res;
    }
    __syncthreads();
    return res;
}

// The chunk holding u * W from chunk sums W[0..splits) in LDS (wave 0 finds
// it; every thread gets it): *chunk and the remaining target *rem inside it
// (INFINITY when rounding left u * W past every running sum: then the last
// chunk with weight, whose last positive entry is drawn).  Returns false if
// the total is not a usable positive number.
__device__ bool pick_chunk(const ChainParams& P, const double* W, double u, int* chunk, double* rem)
{
    __shared__ int32_t sh_chunk;
    __shared__ double sh_t;
    __shared__ int32_t sh_ok;
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        double tot = 0.0;
        for (int s0 = 0; s0 < P.splits; s0 += kWave) tot += (s0 + lane < P.splits) ? W[s0 + lane] : 0.0;
        tot = wave_bcast_f64(wave_incl_f64(tot), kWave - 1);
        const double t = u * tot;
        double carry = 0.0;
        int found = -1, lastpos = -1;
        double before = 0.0;
        for (int s0 = 0; s0 < P.splits && found < 0; s0 += kWave) {
            const double x = (s0 + lane < P.splits) ? W[s0 + lane] : 0.0;
            const double inc = wave_incl_f64(x);
            const uint64_t hit = __ballot(s0 + lane < P.splits && carry + inc > t);
            const uint64_t pos = __ballot(s0 + lane < P.splits && x > 0.0);
            if (pos) lastpos = s0 + 63 - (int)__builtin_clzll(pos);
            if (hit) {
                const int l = (int)__builtin_ctzll(hit);
                found = s0 + l;
                before = carry + wave_bcast_f64(inc - x, l);
            }
            carry += wave_bcast_f64(inc, kWave - 1);
        }
        if (lane == 0) {
            sh_ok = tot > 0.0 && tot < INFINITY && (found >= 0 || lastpos >= 0);
            sh_chunk = found >= 0 ? found : (lastpos >= 0 ? lastpos : 0);
            sh_t = found >= 0 ? t - before : INFINITY;
        }
    }
    __syncthreads();
    *chunk = sh_chunk;
    *rem = sh_t;
    return sh_ok != 0;
}

// Draw with chunk sums W[0..splits) (fp64, in LDS): pick the chunk holding
// u * W, rescan it.  Returns the token, or -1 if the total is unusable.
template <int DTT, int DTD>
__device__ int32_t draw_from_chunks(const ChainParams& P, const Draw& d, const double* W, double u)
{
    int c;
    double rem;
    if (!pick_chunk(P, W, u, &c, &rem)) return -1;
    const int64_t lo = (int64_t)c * P.chunk;
    const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
    return (int32_t)search_range<DTT, DTD>(P, d, lo, hi, rem);
}

// Draw from p of the draw's target row (fallback when a residual has no mass):
// chunk sums recomputed over the whole row into W, then the usual draw.
template <int DTT, int DTD>
__device__ int32_t draw_from_p(const ChainParams& P, const Draw& d, double* W, double u)
{
    Draw d1 = d;
    d1.mode = 1;
    for (int s = 0; s < P.splits; ++s) {
        const int64_t lo = (int64_t)s * P.chunk;
        const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
        const double x = range_sum<DTT, DTD>(P, d1, lo, hi);
        if (threadIdx.x == 0) W[s] = x;
        __syncthreads();
    }
    return draw_from_chunks<DTT, DTD>(P, d1, W, u);
}

// Appends the emitted tokens (the accepted slot tokens `toks`, already in
// LDS, then token `last` at position nacc) at ctx_len[r] = len and writes the
// new length.
__device__ void commit(const ChainParams& P, int r, int n, int nacc, const int32_t* toks, int32_t last, int32_t len,
                       uint32_t* fl)
{
    const bool ok = (len >= 0 && len + n <= P.ctx_cap);
    if (ok) {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
            const int32_t tok = (i == nacc) ? last : toks[i];
            P.ctx[(int64_t)r * P.ctx_stride + len + i] = tok;
        }
    } else if (threadIdx.x == 0) {
        *fl |= SPEC_FLAG_CTX_OVERFLOW;
    }
    if (threadIdx.x == 0) P.ctx_len_out[r] = ok ? len + n : len;
}

// Residual chunk sums.  The K workgroups of a request split its chunks (chunk
// c goes to workgroup c mod K) and stream the target and draft rows of the
// draw: each thread takes kVecs 16-byte vectors of each chunk (vectors t and
// t + kDBlock ...), kRound chunks per round, the next round's loads in flight
// while a round is summed (two register buffers, the loop body twice).  A
// chunk's sum goes out as an agent-scope store; once every store of the
// workgroup has completed, one agent-scope count per workgroup reports them,
// and the workgroup that brings the count to K draws.  Rows of one dtype,
// 16-byte aligned, vocabulary a multiple of a vector.
constexpr int kVecs = kChunkBytes / 16 / kDBlock;   // vectors per thread per chunk
constexpr int kRound = 1;                           // chunks per round

template <int DT>
__device__ __forceinline__ void residual_issue(const char* tp, const char* dp, const ChainParams& P, int c0, int step,
                                               int t, uint4* a, uint4* b)
{
    constexpr int VEC = vec_of<DT>();
    constexpr int ES = DT == SPEC_F32 ? 4 : 2;
#pragma unroll
    for (int u = 0; u < kRound; ++u)
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
            const int64_t e = (int64_t)(c0 + u * step) * P.chunk + (int64_t)(t + v * kDBlock) * VEC;
            const int64_t eo = e < P.vocab ? e : 0;   // past the row: its first vector, unused
            a[u * kVecs + v] = load_stream(tp + eo * ES);
            b[u * kVecs + v] = load_stream(dp + eo * ES);
        }
    // keep the scheduler from hoisting the previous round's arithmetic above
    // these loads (which would wait for everything in flight first)
    __builtin_amdgcn_sched_barrier(0);
}

// Residual weight sum of one 16-byte vector pair: max(0, ep - eq Zt/Zd) per
// entry in fp32, added in entry order.  The final search recomputes exactly
// this arithmetic, so its running sums agree with the published ones.
template <int DT>
__device__ __forceinline__ float residual_vec(const ChainParams& P, const Draw& d, float r32, const uint4& a,
                                              const uint4& b, float* run = nullptr)
{
    constexpr int VEC = vec_of<DT>();
    float z[VEC], x[VEC];
    unpack<DT>(a, z);
    unpack<DT>(b, x);
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        const float ep = fast_exp2(fmaf(z[k], P.c, -d.Ot));
        const float eq = fast_exp2(fmaf(x[k], P.c, -d.Od));
        acc += fmaxf(fmaf(-eq, r32, ep), 0.0f);
        if (run) run[k] = acc;
    }
    return acc;
}

// Sums one round (every register of both buffers is read) into the wave
// slots: one sum per (chunk, vector slot) and wave, i.e. per block of 64
// consecutive vectors.
template <int DT>
__device__ __forceinline__ void residual_round(const ChainParams& P, const Draw& d, int c0, int step, int t,
                                               const uint4* a, const uint4* b, double (*red)[kRound * kVecs])
{
    constexpr int VEC = vec_of<DT>();
    const int lane = t % kWave, wid = t / kWave;
    const float r32 = (float)d.ratio;
    double part[kRound * kVecs];
#pragma unroll
    for (int u = 0; u < kRound; ++u)
#pragma unroll
        for (int v = 0; v < kVecs; ++v) {
            const float w = residual_vec<DT>(P, d, r32, a[u * kVecs + v], b[u * kVecs + v]);
            const int64_t e = (int64_t)(c0 + u * step) * P.chunk + (int64_t)(t + v * kDBlock) * VEC;
            part[u * kVecs + v] = wave_total_f64(e < P.vocab ? (double)w : 0.0);
        }
    if (lane == kWave - 1)
#pragma unroll
        for (int i = 0; i < kRound * kVecs; ++i) red[wid][i] = part[i];
}

// This workgroup's residual sums of request r, published as kSubSums per
// chunk (block q = v * kDWaves + w covers vectors [v * kDBlock + 64 w, + 64)
// of the chunk, so q runs in entry order); returns true in the workgroup that
// completes the request's count.  Workgroup kk takes chunks kk and kk + K,
// then hands out the rest from the request's counter (2K, 2K + 1, ...), one
// chunk ahead, so the K workgroups finish together; the counter is zeroed by
// the statistics pass.
template <int DT>
__device__ bool residual_publish(const ChainParams& P, const Draw& d, int r, int kk, int K)
{
    static_assert(kVecs * kDBlock * 16 == kChunkBytes, "whole vectors per thread per chunk");
    static_assert(kVecs * kDWaves == kSubSums, "one residual sum per wave and vector slot");
    static_assert(kRound == 1, "one chunk per round");
    __shared__ double red[2][kDWaves][kVecs];
    __shared__ int32_t sNext[2];
    __shared__ int32_t sLast;
    const int t = threadIdx.x;
    const char* tp = (const char*)row_ptr<DT>(P.logits, d.row_t, P.stride);
    const char* dp = (const char*)row_ptr<DT>(P.dlogits, d.row_d, P.dstride);
    uint32_t* grab = P.done + P.bs + r;
    // chunk c's sums from the wave slots, after the barrier that follows its round
    auto finish = [&](int c, int par) {
        const int q = t;
        if (q < kSubSums && c < P.splits) {
            const double sum = red[par][q % kDWaves][q / kDWaves];
            __hip_atomic_store(&P.sums[((int64_t)r * P.splits + c) * kSubSums + q], sum, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    uint4 a0[kVecs], b0[kVecs], a1[kVecs], b1[kVecs];
    int c0 = kk, c1 = kk + K;
    residual_issue<DT>(tp, dp, P, c0, K, t, a0, b0);
    uint32_t g = 0;
    if (t == 0) g = __hip_atomic_fetch_add(grab, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // rounds alternate between buffers 0 and 1 and between red[0] and red[1],
    // so one barrier per round suffices (chunks past the row read first
    // vectors and publish nothing)
    while (c0 < P.splits) {
        residual_issue<DT>(tp, dp, P, c1, K, t, a1, b1);
        residual_round<DT>(P, d, c0, K, t, a0, b0, red[0]);
        if (t == 0) sNext[0] = 2 * K + (int)g;
        __syncthreads();
        finish(c0, 0);
        const int c2 = sNext[0];
        if (t == 0) g = __hip_atomic_fetch_add(grab, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        residual_issue<DT>(tp, dp, P, c2, K, t, a0, b0);
        residual_round<DT>(P, d, c1, K, t, a1, b1, red[1]);
        if (t == 0) sNext[1] = 2 * K + (int)g;
        __syncthreads();
        finish(c1, 1);
        c0 = c2;
        c1 = sNext[1];
        if (t == 0 && c0 < P.splits) g = __hip_atomic_fetch_add(grab, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    drain(a0);
    drain(b0);
    // every sum store of the workgroup completes before the count reports them
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
        const uint32_t before = __hip_atomic_fetch_add(&P.done[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sLast = before + 1 == (uint32_t)K;
    }
    __syncthreads();
    return sLast != 0;
}

// One published residual sum; a sum still -1 is not yet visible and is read
// again, at most `limit` more times (in practice it never spins).  Returns -1
// if the sum did not arrive (limit < 0: without reading it at all).
__device__ __forceinline__ double residual_load(const double* w, int32_t limit)
{
    if (limit < 0) return -1.0;
    double v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int32_t tries = 0; v < 0.0 && tries < limit; ++tries)
        v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
}

// Draw of a streamed residual (the drawing workgroup; splits <= kDBlock):
// thread s gathers chunk s's published sums, the chunk is picked from their
// totals, then wave 0 picks the block of 64 vectors from the chunk's
// kSubSums and finds the entry among the block's 64 x VEC with one load of
// both rows per lane.  Returns the token, -1 if the residual has no usable
// mass, or kResidualLate if a published sum did not arrive within the bounded
// wait (the caller then sums the residual itself).
constexpr int32_t kResidualLate = -2;

template <int DT>
__device__ int32_t residual_draw(const ChainParams& P, const Draw& d, int r, double u, double* W)
{
    constexpr int VEC = vec_of<DT>();
    constexpr int ES = DT == SPEC_F32 ? 4 : 2;
    __shared__ double sSub[kSubSums];
    __shared__ int32_t sTok;
    __shared__ int32_t sLate;
    const int t = threadIdx.x;
    double mine[kSubSums];
    if (t == 0) sLate = 0;
    __syncthreads();
    if (t < P.splits) {
        const double* src = P.sums + ((int64_t)r * P.splits + t) * kSubSums;
        // every sum of the chunk in one round trip; a sum not yet visible
        // (never seen in practice) is then waited for on its own
        bool missing = P.wait_limit < 0;
        if (!missing) {
#pragma unroll
            for (int q = 0; q < kSubSums; ++q)
                mine[q] = __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int q = 0; q < kSubSums; ++q) missing |= mine[q] < 0.0;
        }
        if (missing) {
            // the rare case: wait for each sum in turn, within the bound
#pragma unroll
            for (int q = 0; q < kSubSums; ++q) mine[q] = residual_load(src + q, P.wait_limit);
        }
        double tot = 0.0;
        bool late = false;
#pragma unroll
        for (int q = 0; q < kSubSums; ++q) {
            late |= mine[q] < 0.0;
            tot += mine[q];
        }
        W[t] = tot;
        if (late) sLate = 1;
    }
    __syncthreads();
    if (sLate) return kResidualLate;
    int c;
    double rem;
    if (!pick_chunk(P, W, u, &c, &rem)) return -1;
    if (t == c)
#pragma unroll
        for (int q = 0; q < kSubSums; ++q) sSub[q] = mine[q];
    __syncthreads();
    if (t < kWave) {
        const int lane = t;
        // the block of the chunk: inclusive running sums over kSubSums lanes
        const double x = lane < kSubSums ? sSub[lane] : 0.0;
        const double inc = wave_incl_f64(x);
        const uint64_t hit = __ballot(lane < kSubSums && inc > rem);
        const uint64_t pos = __ballot(lane < kSubSums && x > 0.0);
        const int q = hit ? (int)__builtin_ctzll(hit) : (pos ? 63 - (int)__builtin_clzll(pos) : 0);
        const double remq = hit ? rem - wave_bcast_f64(inc - x, q) : INFINITY;
        // lane l: vector v * kDBlock + 64 w + l of chunk c, both rows
        const int v = q / kDWaves, w = q % kDWaves;
        const int64_t e = (int64_t)c * P.chunk + ((int64_t)v * kDBlock + 64 * w + lane) * VEC;
        const int64_t eo = e < P.vocab ? e : 0;
        const uint4 a = *(const uint4*)((const char*)row_ptr<DT>(P.logits, d.row_t, P.stride) + eo * ES);
        const uint4 b = *(const uint4*)((const char*)row_ptr<DT>(P.dlogits, d.row_d, P.dstride) + eo * ES);
        float run[VEC];
        float wl = residual_vec<DT>(P, d, (float)d.ratio, a, b, run);
        if (e >= P.vocab) {
            wl = 0.0f;
#pragma unroll
            for (int k = 0; k < VEC; ++k) run[k] = 0.0f;
        }
        // running sum over the lanes (fp64), then the first lane that passes
        const double li = wave_incl_f64((double)wl);
        const double before = li - (double)wl;
        const uint64_t cross = __ballot(wl > 0.0f && li > remq);
        const uint64_t lpos = __ballot(wl > 0.0f);
        // the entry: the first of the lane whose running sum passes, else (rounding) its last positive one
        auto entry = [&](bool search) {
            int k = -1;
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
                const bool positive = run[j] > (j ? run[j - 1] : 0.0f);
                if (positive && (k < 0 || !search) && (!search || before + (double)run[j] > remq)) k = j;
            }
            if (k < 0)
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (run[j] > (j ? run[j - 1] : 0.0f)) k = j;
            return (int32_t)(e + (k < 0 ? 0 : k));
        };
        if (cross) {
            if (lane == (int)__builtin_ctzll(cross)) sTok = entry(true);
        } else if (lpos) {
            if (lane == 63 - (int)__builtin_clzll(lpos)) sTok = entry(false);   // rounding: the block's last positive entry
        } else if (lane == 0) {
            sTok = -1;
        }
    }
    __syncthreads();
    return sTok;
}

// ---------------------------------------------------------------------------
// decide, draw, commit: one workgroup per request
// ---------------------------------------------------------------------------

constexpr int kMaxPartsLds = 2176;   // partials of one request staged in LDS (34 KB)
// The fused n-gram scan takes 17 positions per thread per batch: its window
// (8,704 tokens, in the partials' LDS) holds a context of 8,192 tokens and
// the tokens one step appends, so such a text needs one batch.
constexpr int kNgBatch = 17;

constexpr int kMergeLanes = 8;   // lanes that merge one row's chunk partials

// Grid (bs, K): the K workgroups of a request all merge its partials and find
// the first rejection (cheap, and identical); workgroup 0 writes the slot
// outputs and draws and commits, except that a probabilistic residual is
// summed by all K and drawn by the last of them to finish.
template <int DTT, int DTD>
__global__ __launch_bounds__(kDBlock) void k_decide(ChainParams P)
{
    const int r = blockIdx.x;
    const int kk = blockIdx.y, K = gridDim.y;
    const bool lead = kk == 0;
    const int t = threadIdx.x;
    const int ld = P.ld;
    const int32_t len0 = P.ctx ? P.ctx_len[r] : 0;   // loaded early, used by the commit
    const double usmp = P.greedy ? 0.0 : (P.rng ? (double)step_uniform(P, r, SPEC_MAX_DRAFT) : (double)P.u_smp[r]);
    __shared__ Partial sp[kMaxPartsLds];
    __shared__ float sO[2 * SPEC_MAX_DRAFT + 1];
    __shared__ double sZ[2 * SPEC_MAX_DRAFT + 1];
    __shared__ int32_t sArg[2 * SPEC_MAX_DRAFT + 1];
    __shared__ int32_t sOk[2 * SPEC_MAX_DRAFT + 1];
    __shared__ int32_t sTok[SPEC_MAX_DRAFT];
    __shared__ uint8_t sPm[SPEC_MAX_DRAFT];
    __shared__ double sW[kMaxSplits];
    __shared__ uint32_t sFlags;
    __shared__ unsigned long long sRej;
    __shared__ float sZy;   // target logit of the first rejected slot's token
    // Slot inputs first (thread t = slot t), including the logits of each
    // slot's token, so that these dependent loads overlap the staging and the
    // merges below.
    int b = P.n_slots[r];
    const int64_t row_base = P.row_base[r];
    int32_t y = -1;
    bool pm = true;
    float uacc = 0.0f, zt = 0.0f, zd = 0.0f;
    if (t < ld) {
        const int64_t off = (int64_t)r * ld + t;
        y = P.tokens[off];
        pm = !P.slot_flags || (P.slot_flags[off] & SPEC_SLOT_POINT_MASS);
        const bool yok = y >= 0 && y < P.vocab;
        if (!P.greedy) {
            uacc = P.rng ? step_uniform(P, r, t) : P.u_acc[off];
            const int64_t row = row_base + t;
            if (yok && row >= 0 && row < P.n_rows) zt = logit_at(P.logits, DTT, row, P.stride, y);
            if (!pm && P.dlogits) {
                const int64_t drow = P.drow_base[r] + t;
                if (yok && drow >= 0 && drow < P.dn_rows) zd = logit_at(P.dlogits, P.ddt, drow, P.dstride, y);
            }
        }
        sTok[t] = y;
        sPm[t] = pm;
    }
    const bool badlen = (b < 0 || b > ld);
    b = b < 0 ? 0 : (b > ld ? ld : b);
    if (t == 0) { sFlags = badlen ? SPEC_FLAG_BAD_LENGTH : 0u; sRej = 0; }
    // stage this request's partials (contiguous) in LDS, split-major
    // (sp[s * NR + row])
    const int nparts = P.NR * P.splits;
    const bool staged = nparts <= kMaxPartsLds;
    const Partial* gp = P.part + (int64_t)r * nparts;
    if (staged)
        for (int i = t; i < nparts; i += kDBlock) {
            const int row = i / P.splits, s = i - row * P.splits;
            sp[s * P.NR + row] = gp[i];
        }
    __syncthreads();
    // Rows: target 0..b, draft ld+1 .. ld+b (probabilistic slots, T > 0).
    // kMergeLanes lanes merge one row: each folds every kMergeLanes-th chunk
    // partial online, then the lanes combine pairwise. The merge is
    // instantiated once for LDS partials and once for global ones, so that
    // each reads through its own address space (a pointer that may be either
    // compiles to flat loads, which wait for every outstanding access).
    // rs: stride between a row's splits; rr: between rows.
    auto merge = [&](const auto* rp, int rs, int rr) __attribute__((always_inline)) {
    for (int row0 = 0; row0 < P.NR; row0 += kDBlock / kMergeLanes) {
        const int row = row0 + t / kMergeLanes, j = t % kMergeLanes;
        bool is_row = row < P.NR && row <= b;
        if (!is_row && row < P.NR && !P.greedy && P.dlogits && row >= ld + 1 && row <= ld + b)
            is_row = !sPm[row - ld - 1];
        if (P.greedy) {
            ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
            if (is_row)
                for (int s = j; s < P.splits; s += kMergeLanes) {
                    const Partial q = rp[row * rr + s * rs];
                    ArgAcc bq{q.m, q.idx & 0x7FFFFFFF, (q.idx >> 31) & 1};
                    if (q.m != q.m) bq.bad = 1;
                    am_combine(acc, bq);
                }
#pragma unroll
            for (int o = 1; o < kMergeLanes; o <<= 1) {
                ArgAcc bq{__shfl_xor(acc.best, o, kWave), __shfl_xor(acc.idx, o, kWave), __shfl_xor(acc.bad, o, kWave)};
                am_combine(acc, bq);
            }
            if (j == 0 && row < P.NR) {
                sOk[row] = is_row && !acc.bad && acc.idx != 0x7FFFFFFF;
                sArg[row] = acc.idx;
            }
        } else {
            float m = -INFINITY;
            double z = 0.0;
            int nan = 0;
            if (is_row)
                for (int s = j; s < P.splits; s += kMergeLanes) {
                    const Partial q = rp[row * rr + s * rs];
                    nan |= (q.m != q.m) || (q.s != q.s);
                    if (q.m == -INFINITY) continue;
                    if (q.m > m) {
                        if (m != -INFINITY) z *= (double)fast_exp2((float)((double)(m * P.c) - (double)(q.m * P.c)));
                        m = q.m;
                    }
                    z += q.s * (double)fast_exp2((float)((double)(q.m * P.c) - (double)(m * P.c)));
                }
#pragma unroll
            for (int o = 1; o < kMergeLanes; o <<= 1) {
                const float m2 = __shfl_xor(m, o, kWave);
                const double z2 = __shfl_xor(z, o, kWave);
                nan |= __shfl_xor(nan, o, kWave);
                sm_combine(m, z, m2, z2, P.c);
            }
            if (j == 0 && row < P.NR) {
                sOk[row] = is_row && !nan && m != -INFINITY && m != INFINITY && z > 0.0 && z < INFINITY;
                sO[row] = m * P.c;
                sZ[row] = z;
            }
        }
    }
    };
    if (staged) merge(sp, P.NR, 1);
    else merge(gp, 1, P.splits);
    __syncthreads();
    // slot i = t < b: p(y), q(y), accept
    bool rejected = false;
    uint32_t slot_fl = 0;
    if (t < b) {
        bool acc = true;
        uint32_t fl = 0;
        const int64_t off = (int64_t)r * ld + t;
        const bool bad = (y < 0 || y >= P.vocab);
        if (bad) fl |= SPEC_FLAG_BAD_TOKEN;
        if (!sOk[t]) fl |= SPEC_FLAG_BAD_LOGITS;
        double p = 0.0, q = 1.0;
        if (P.greedy) {
            p = (!bad && sOk[t] && sArg[t] == y) ? 1.0 : 0.0;
            acc = (p == 1.0);
        } else {
            if (!bad && sOk[t]) p = (double)fast_exp2(fmaf(zt, P.c, -sO[t])) / sZ[t];
            if (!pm) {
                const int dr = ld + 1 + t;
                if (!sOk[dr]) fl |= SPEC_FLAG_BAD_LOGITS;
                q = 0.0;
                if (!bad && sOk[dr] && P.dlogits) q = (double)fast_exp2(fmaf(zd, P.c, -sO[dr])) / sZ[dr];
            }
            const double rho = q > 0.0 ? p / q : 0.0;
            acc = (double)uacc < rho;
        }
        if (P.out_p && lead) P.out_p[(int64_t)r * (ld + 1) + t] = (float)p;
        if (P.out_q && lead) P.out_q[off] = (float)q;
        rejected = !acc;
        slot_fl = fl;
    } else if (t <= ld && lead) {
        // past the slots; entry b of out_p (the bonus row) is the drawing
        // workgroup's to write
        if (P.out_p && t != b) P.out_p[(int64_t)r * (ld + 1) + t] = 0.0f;
        if (P.out_q && t < ld) P.out_q[(int64_t)r * ld + t] = 0.0f;
    }
    // every slot thread is in wave 0 (b <= ld <= 32): a ballot and an OR
    // across the wave instead of atomics
    if (t < kWave) {
        const uint64_t rj = __ballot(rejected);
        const uint32_t f = wave_or(slot_fl);
        if (t == 0) {
            sRej = rj;
            sFlags |= f;
        }
    }
    __syncthreads();
    const uint64_t rej = sRej;
    const int nacc = rej ? (int)__builtin_ctzll(rej) : b;
    if (t == nacc && t < b) sZy = zt;   // read after the next barrier
    // token nacc (the correction or bonus) is written by the drawing
    // workgroup alone, which need not be this one
    if (lead && t <= ld && t != nacc) P.out_tokens[(int64_t)r * (ld + 1) + t] = (t < nacc) ? y : -1;
    if (t == 0) {
        if (lead) {
            P.out_num[r] = nacc + 1;
            P.out_acc[r] = nacc;
            if (P.accept_hist) atomicAdd(&P.accept_hist[nacc], 1);
        }
        if (nacc == b && !sOk[b]) sFlags |= SPEC_FLAG_BAD_LOGITS;
    }
    // what to draw
    Draw d;
    d.mode = 0; d.y = -1; d.Ot = d.Od = 0.0f; d.row_t = row_base + nacc; d.row_d = -1; d.ratio = 1.0;
    int32_t last = -1;
    if (P.greedy) {
        last = sOk[nacc] ? sArg[nacc] : -1;
        if (last == 0x7FFFFFFF) last = -1;
    } else if (sOk[nacc] && d.row_t >= 0 && d.row_t < P.n_rows) {
        d.Ot = sO[nacc];
        if (nacc == b) {
            d.mode = 1;
        } else {
            const int32_t yn = sTok[nacc];
            const bool pmn = sPm[nacc];
            const bool bad = (yn < 0 || yn >= P.vocab);
            const int dr = ld + 1 + nacc;
            if (bad) d.mode = 1;
            else if (pmn) { d.mode = 3; d.y = yn; }
            else if (sOk[dr] && P.dlogits) {
                d.mode = 2; d.y = yn; d.row_d = P.drow_base[r] + nacc; d.Od = sO[dr]; d.ratio = sZ[nacc] / sZ[dr];
            } else d.mode = 1;   // unusable draft row (flagged): fall back to p
        }
    }
    double* W = sW;   // chunk sums of the draw
    // which workgroup draws: the lead, or for a streamed residual the last
    // of the K to finish its chunks
    bool streamed = false;
    if constexpr (DTT == DTD) streamed = d.mode == 2 && P.coal && P.splits <= kDBlock;
    if (streamed) {
        const bool drawer = residual_publish<DTT>(P, d, r, kk, K);
        if (!drawer) {
            // the drawing workgroup reports the request's flags (it has them all)
            return;
        }
    } else if (!lead) {
        return;
    }
    // the first batch of the n-gram window (the request's text before the
    // commit), in flight while the draw runs; the committed tokens are
    // patched in afterwards
    int32_t ngv[kNgBatch];
    if (P.ng_draft) {
        const int32_t* row = P.ctx + (int64_t)r * P.ctx_stride;
        const int64_t lastp = P.ctx_stride - 1;   // >= 0 (checked by the host)
#pragma unroll
        for (int u = 0; u < kNgBatch; ++u) {
            const int64_t j = t + (int64_t)u * kDBlock;
            ngv[u] = row[j < lastp ? j : lastp];
        }
    }
    bool resum = false;   // a streamed residual whose published sums did not all arrive
    bool zero = false;    // the residual had no mass (not reachable in exact arithmetic)
    if (streamed) {
        last = residual_draw<DTT>(P, d, r, usmp, W);
        if (last == kResidualLate) {
            if (t == 0) sFlags |= SPEC_FLAG_RESIDUAL_LATE;
            resum = true;
        } else if (last < 0) {
            zero = true;
        }
    }
    if (!streamed || resum) {
      if (d.mode != 0) {
        if (d.mode == 2) {
            // residual max(0, p - q) of rows that do not take the vector path: chunk by chunk
            for (int s = 0; s < P.splits; ++s) {
                const int64_t lo = (int64_t)s * P.chunk;
                const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
                const double x = range_sum<DTT, DTD>(P, d, lo, hi);
                if (t == 0) W[s] = x;
            }
            __syncthreads();
        } else {
            // chunk sums of the row from its partials; for a point-mass
            // residual, y's chunk without y
            auto sums = [&](const auto* row, int rs) __attribute__((always_inline)) {
                for (int s = t; s < P.splits; s += kDBlock) {
                    const Partial q = row[s * rs];
                    W[s] = (q.m == -INFINITY) ? 0.0 : q.s * (double)fast_exp2((float)((double)(q.m * P.c) - (double)d.Ot));
                }
            };
            if (staged) sums(sp + nacc, P.NR);
            else sums(gp + nacc * P.splits, 1);
            __syncthreads();
            if (d.mode == 3) {
                // Subtract y's term from its chunk's sum when that leaves at
                // least half of the sum (the cancellation then costs at most
                // one bit); otherwise rescan the chunk without y.
                const int sy = (int)(d.y / P.chunk);
                const double cs = W[sy];
                const double wy = (double)fast_exp2(fmaf(sZy, P.c, -d.Ot));
                if (wy <= 0.5 * cs) {
                    __syncthreads();
                    if (t == 0) W[sy] = cs - wy;
                } else {
                    const int64_t lo = (int64_t)sy * P.chunk;
                    const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
                    const double w = range_sum<DTT, DTD>(P, d, lo, hi);
                    if (t == 0) W[sy] = w;
                }
            }
            __syncthreads();
        }
        last = draw_from_chunks<DTT, DTD>(P, d, W, usmp);
        zero = last < 0;
      } else if (!P.greedy) {
        if (t == 0) sFlags |= SPEC_FLAG_BAD_LOGITS;
      }
    }
    if (zero) {
        // a residual without mass: draw from p (one call site, so that it is inlined)
        if (t == 0) sFlags |= SPEC_FLAG_RESIDUAL_ZERO;
        last = draw_from_p<DTT, DTD>(P, d, W, usmp);
    }
    if (t == 0) {
        P.out_tokens[(int64_t)r * (ld + 1) + nacc] = last;
        if (P.out_p) {
            // p of the bonus row at the bonus token (0 when a slot was rejected)
            float pb = 0.0f;
            if (nacc == b && last >= 0 && last < P.vocab && sOk[b]) {
                if (P.greedy) pb = 1.0f;
                else if (d.mode == 1)
                    pb = (float)((double)fast_exp2(fmaf(logit_at(P.logits, DTT, d.row_t, P.stride, last), P.c, -d.Ot)) /
                                 sZ[b]);
            }
            P.out_p[(int64_t)r * (ld + 1) + b] = pb;
        }
    }
    __syncthreads();
    uint32_t fl = sFlags;
    if (P.ctx) {
        __shared__ uint32_t sCommit;
        if (t == 0) sCommit = 0;
        __syncthreads();
        commit(P, r, nacc + 1, nacc, sTok, last, len0, &sCommit);
        __syncthreads();
        fl |= sCommit;
    }
    if (t == 0) {
        if (P.write_flags) P.out_flags[r] = fl;
        else if (fl) atomicOr(&P.out_flags[r], fl);
    }
    if (P.ng_draft) {
        // the next n-gram draft over the committed context: its stores are
        // visible to the workgroup after the barrier, and the partials' and
        // chunk sums' LDS is free for the scan's window and lists
        static_assert(sizeof(sp) >= sizeof(int32_t) * kDBlock * kNgBatch, "scan window fits the partials' LDS");
        static_assert(sizeof(sW) >= sizeof(NgramShared<kDBlock>), "scan lists fit the chunk sums' LDS");
        const int32_t n = nacc + 1;
        const bool appended = len0 >= 0 && len0 + n <= P.ctx_cap;   // as the commit decided
        int64_t nl = appended ? (int64_t)len0 + n : (int64_t)len0;
        nl = nl < 0 ? 0 : (nl > P.ctx_stride ? P.ctx_stride : nl);
        if (appended)
#pragma unroll
            for (int u = 0; u < kNgBatch; ++u) {
                const int64_t j = t + (int64_t)u * kDBlock - len0;
                if (j >= 0 && j < n) ngv[u] = j < nacc ? sTok[j] : last;
            }
        Text x;
        x.a = P.ctx + (int64_t)r * P.ctx_stride; x.na = nl; x.b = nullptr; x.n = nl;
        NgramOut O;
        O.n_min = P.ng_min; O.n_max = P.ng_max; O.max_draft = P.ng_ld; O.cap = P.ng_cap;
        O.draft = P.ng_draft + (int64_t)r * P.ng_ld;
        O.draft_len = P.ng_len + r;
        O.feat = P.ng_feat + 4 * (int64_t)r;
        O.follow_ctx = 0;   // the chain drafter copies only
        O.follow = nullptr;
        __syncthreads();
        ngram_scan<kDBlock, kNgBatch>(x, (int32_t*)sp, *(NgramShared<kDBlock>*)sW, O, ngv, true);
    }
}

// ---------------------------------------------------------------------------
// tree walk (greedy)
// ---------------------------------------------------------------------------

struct TreeParams {
    int32_t bs, vocab, rows_max;
    const int32_t* node_token; const int32_t* parent_row; const int32_t* n_rows;
    int32_t* out_tokens; int32_t* out_num; int32_t* out_path; int32_t* out_argmax; uint32_t* out_flags;
    int32_t* ctx; int64_t ctx_stride; const int32_t* ctx_len; int32_t* ctx_len_out; int32_t ctx_cap;
    Partial* part; int32_t splits;
};

template <int kPer>
__global__ __launch_bounds__(kWave) void k_tree_walk(TreeParams P)
{
    const int r = blockIdx.x, t = threadIdx.x;
    const int rm = P.rows_max;
    // the rows' chunk partials (all rows_max rows of the request's slice, so
    // that no load waits for the row count), the row count and the tree are
    // all requested before the first use: one memory round trip in all (kPer
    // partials per lane: the host picks the smaller instance when they fit)
    constexpr int kWalkParts = kPer * kWave;
    __shared__ Partial sp[kWalkParts];
    const int total = rm * P.splits;
    const bool staged = total <= kWalkParts;
    const Partial* gp = P.part + (int64_t)r * rm * P.splits;
    uint4 held[kPer];
    {
        // clamped to the slice's last partial (a repeat that is not stored)
        const uint4* g4 = (const uint4*)gp;
        const int last = (staged ? total : 1) - 1;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = t + u * kWave;
            held[u] = g4[i < last ? i : last];
        }
    }
    int n = P.n_rows[r];
    int32_t tok = -2, par = -2;
    if (t < rm) {
        tok = P.node_token[(int64_t)r * rm + t];
        par = P.parent_row[(int64_t)r * rm + t];
    }
    const bool badlen = (n < 1 || n > rm);
    n = n < 1 ? 1 : (n > rm ? rm : n);
    __shared__ int32_t sArg[SPEC_MAX_ROWS];
    __shared__ int32_t sOk[SPEC_MAX_ROWS];
    __shared__ int32_t sOut[SPEC_MAX_ROWS];
    __shared__ int32_t sPath[SPEC_MAX_ROWS];
    __shared__ int32_t sNum;
    __shared__ uint32_t sFl;
    {
        // every slot is written (those past the slice with its last partial)
        // so that no load sinks into a branch and waits alone
        uint4* s4 = (uint4*)sp;
#pragma unroll
        for (int u = 0; u < kPer; ++u) s4[t + u * kWave] = held[u];
    }
    __syncthreads();
    {
        // each row's partials merged by g lanes, then across them (the merge
        // keeps the largest value and its lowest index, in any grouping); one
        // loop per address space (a pointer that may be either compiles to
        // flat loads)
        const int lg = n <= kWave / 4 ? 2 : (n <= kWave / 2 ? 1 : 0), g = 1 << lg;
        const int row = t >> lg, sub = t & (g - 1);
        ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
        auto take = [&](const Partial q) {
            ArgAcc b{q.m, q.idx & 0x7FFFFFFF, (q.idx >> 31) & 1};
            if (q.m != q.m) b.bad = 1;
            am_combine(acc, b);
        };
        if (row < n) {
            if (staged)
                for (int s = sub; s < P.splits; s += g) take(sp[(int64_t)row * P.splits + s]);
            else
                for (int s = sub; s < P.splits; s += g) take(gp[(int64_t)row * P.splits + s]);
        }
        for (int o = 1; o < g; o <<= 1) {
            ArgAcc b{__shfl_xor(acc.best, o, kWave), __shfl_xor(acc.idx, o, kWave), __shfl_xor(acc.bad, o, kWave)};
            am_combine(acc, b);
        }
        if (row < n && sub == 0) {
            sOk[row] = !acc.bad && acc.idx != 0x7FFFFFFF;
            sArg[row] = (acc.idx == 0x7FFFFFFF) ? -1 : acc.idx;
        }
    }
    for (int i = t; i < rm; i += kWave) { sOut[i] = -1; sPath[i] = -1; }
    __syncthreads();
    // the path, one step per ballot: lane c holds row c's parent and token
    // (rows_max <= 64, one wave), and the lowest matching child is taken
    {
        const int myPar = t < n ? par : -2, myTok = t < n ? tok : -2;
        const uint64_t bad = __ballot(t < n && !sOk[t]);
        int u = 0, k = 0;
        if (t == 0) sPath[0] = 0;
        for (;;) {
            const int a = sArg[u];
            const uint64_t hit = __ballot(t >= 1 && t < n && myPar == u && myTok == a);
            if (t == 0) sOut[k] = a;
            ++k;
            if (!hit || k >= rm) break;
            u = (int)__builtin_ctzll(hit);
            if (t == 0) sPath[k] = u;
        }
        if (t == 0) {
            sNum = k;
            sFl = (badlen ? SPEC_FLAG_BAD_LENGTH : 0u) | (bad ? SPEC_FLAG_BAD_LOGITS : 0u);
        }
    }
    __syncthreads();
    for (int i = t; i < rm; i += kWave) {
        P.out_tokens[(int64_t)r * rm + i] = sOut[i];
        P.out_path[(int64_t)r * rm + i] = sPath[i];
        if (P.out_argmax) P.out_argmax[(int64_t)r * rm + i] = (i < n) ? sArg[i] : -1;
    }
    if (t == 0) P.out_num[r] = sNum;
    uint32_t fl = sFl;
    if (P.ctx) {
        const int32_t len = P.ctx_len[r];
        const bool ok = (len >= 0 && len + sNum <= P.ctx_cap);
        if (ok) {
            for (int i = t; i < sNum; i += kWave) P.ctx[(int64_t)r * P.ctx_stride + len + i] = sOut[i];
        } else {
            fl |= SPEC_FLAG_CTX_OVERFLOW;
        }
        __syncthreads();
        if (t == 0) P.ctx_len_out[r] = ok ? len + sNum : len;
    }
    if (t == 0 && fl) atomicOr(&P.out_flags[r], fl);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

static bool aligned16(const void* p, int64_t stride, int dt)
{
    const int64_t es = dt == SPEC_F32 ? 4 : 2;
    return ((uintptr_t)p % 16 == 0) && ((stride * es) % 16 == 0);
}

// Upper bound of the statistics items (the exact count is on the device).
static int64_t stats_items(int32_t bs, int rows_per_req_max, const RowSplit& sp)
{
    return (int64_t)bs * rows_per_req_max * sp.splits;
}

// The only state the library keeps between calls: caches of device
// properties that never change while the process runs (compute units per
// device, workgroups per compute unit per kernel), filled on first use under
// a lock, in fixed-size tables (no heap allocation on any launch path).
static std::mutex g_cache_mu;

// Compute units of the current device (cached per device).
static int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(g_cache_mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Workgroups of `block` threads that one compute unit holds at once (cached
// per kernel; the kernels' resource use is the same on every gfx950 device).
static int blocks_per_cu(const void* kernel, int block)
{
    static const void* keys[256];
    static int vals[256];
    static int used = 0;
    std::lock_guard<std::mutex> lock(g_cache_mu);
    for (int i = 0; i < used; ++i)
        if (keys[i] == kernel) return vals[i];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess || n <= 0) n = 1;
    if (used < 256) {
        keys[used] = kernel;
        vals[used] = n;
        ++used;
    }
    return n;
}

// One resident wave of workgroups (a second round would only add a tail),
// at most one per unit of work.
static int resident_grid(const void* kernel, int block, int64_t work)
{
    const int64_t cap = (int64_t)blocks_per_cu(kernel, block) * device_cus();
    const int64_t g = work < cap ? work : cap;
    return (int)(g > 0 ? g : 1);
}

// Stream plus the optional event pair that brackets the statistics kernel
// itself (attached to its dispatch, so the pair times exactly that kernel).
struct StatsLaunch {
    hipStream_t st;
    hipEvent_t e0, e1;
};

template <typename K>
static void launch_timed(K kern, int grid, int block, const StatsParams& P, const StatsLaunch& L)
{
    if (L.e0 || L.e1)
        hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, L.st, L.e0, L.e1, 0, P);
    else
        hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, L.st, P);
}

template <int DT, bool A, int DDT, bool DA, bool GREEDY, bool DRAFT, bool GPRE>
static void launch_stats_t(const StatsParams& P, int64_t items, const StatsLaunch& L)
{
    constexpr int VEC = A ? vec_of<DT>() : 1;
    constexpr int DVEC = DA ? vec_of<DDT>() : 1;
    auto kern = k_stats<DT, VEC, DDT, DVEC, GREEDY, DRAFT, GPRE>;
    launch_timed(kern, resident_grid((const void*)kern, kBlock, items), kBlock, P, L);
}

template <int DT, bool A, bool GREEDY, bool GPRE>
static void launch_stats_d(const StatsParams& P, int ddt, bool da, bool draft, int64_t items, const StatsLaunch& st)
{
    if (!draft) { launch_stats_t<DT, A, SPEC_F32, false, GREEDY, false, GPRE>(P, items, st); return; }
    if (ddt == SPEC_F32) {
        if (da) launch_stats_t<DT, A, SPEC_F32, true, GREEDY, true, GPRE>(P, items, st);
        else launch_stats_t<DT, A, SPEC_F32, false, GREEDY, true, GPRE>(P, items, st);
    } else {
        if (da) launch_stats_t<DT, A, SPEC_BF16, true, GREEDY, true, GPRE>(P, items, st);
        else launch_stats_t<DT, A, SPEC_BF16, false, GREEDY, true, GPRE>(P, items, st);
    }
}

template <bool GREEDY, bool GPRE>
static void launch_stats_g(const StatsParams& P, int dt, bool a, int ddt, bool da, bool draft, int64_t items,
                           const StatsLaunch& st)
{
    if (dt == SPEC_F32) {
        if (a) launch_stats_d<SPEC_F32, true, GREEDY, GPRE>(P, ddt, da, draft, items, st);
        else launch_stats_d<SPEC_F32, false, GREEDY, GPRE>(P, ddt, da, draft, items, st);
    } else {
        if (a) launch_stats_d<SPEC_BF16, true, GREEDY, GPRE>(P, ddt, da, draft, items, st);
        else launch_stats_d<SPEC_BF16, false, GREEDY, GPRE>(P, ddt, da, draft, items, st);
    }
}

template <int DT, int DDT, bool DA, bool GREEDY, int DMODE>
static void launch_pipe_t(const StatsParams& P, int64_t items, const StatsLaunch& L)
{
    constexpr int DVEC = DA ? vec_of<DDT>() : 1;
    auto kern = k_stats_pipe<DT, DDT, DVEC, GREEDY, DMODE>;
    launch_timed(kern, resident_grid((const void*)kern, kPipeBlock, (items + kGroups - 1) / kGroups), kPipeBlock, P,
                 L);
}

template <int DT, bool GREEDY>
static void launch_pipe_d(const StatsParams& P, int ddt, bool da, bool draft, bool ditems, int64_t items,
                          const StatsLaunch& L)
{
    if (GREEDY || !draft) { launch_pipe_t<DT, SPEC_F32, false, GREEDY, kDraftNone>(P, items, L); return; }
    if constexpr (!GREEDY) {
        if (ditems) { launch_pipe_t<DT, DT, true, false, kDraftItems>(P, items, L); return; }
        if (ddt == SPEC_F32) {
            if (da) launch_pipe_t<DT, SPEC_F32, true, false, kDraftInline>(P, items, L);
            else launch_pipe_t<DT, SPEC_F32, false, false, kDraftInline>(P, items, L);
        } else {
            if (da) launch_pipe_t<DT, SPEC_BF16, true, false, kDraftInline>(P, items, L);
            else launch_pipe_t<DT, SPEC_BF16, false, false, kDraftInline>(P, items, L);
        }
    }
}

template <int DT, bool GREEDY, bool DITEMS>
static void launch_flat_t(const StatsParams& P, int64_t grid, const StatsLaunch& L)
{
    hipLaunchKernelGGL(k_plan_rows<DITEMS>, dim3(1), dim3(kBlock), 0, L.st, P);
    if constexpr (GREEDY) launch_timed(k_stats_flat<DT, GREEDY, DITEMS>, (int)grid, kBlock, P, L);
    else launch_timed(k_stats_flat_half<DT, DITEMS>, (int)grid, kHalf, P, L);
}

template <int DT>
static void launch_flat_d(const StatsParams& P, bool greedy, bool draft, int64_t grid, const StatsLaunch& L)
{
    if (greedy) launch_flat_t<DT, true, false>(P, grid, L);
    else if (draft) launch_flat_t<DT, false, true>(P, grid, L);
    else launch_flat_t<DT, false, false>(P, grid, L);
}

template <int DT, bool GREEDY, bool DITEMS>
static void launch_rows_t(const StatsParams& P, int tm, int dm, const StatsLaunch& L)
{
    const dim3 grid((unsigned)((tm + dm) * ((P.splits + 1) / 2)), (unsigned)P.bs);
    auto kern = k_stats_rows<DT, GREEDY, DITEMS>;
    if (L.e0 || L.e1)
        hipExtLaunchKernelGGL(kern, grid, dim3(kBlock), 0, L.st, L.e0, L.e1, 0, P, (int32_t)tm);
    else
        hipLaunchKernelGGL(kern, grid, dim3(kBlock), 0, L.st, P, (int32_t)tm);
}

template <int DT>
static void launch_rows_d(const StatsParams& P, bool greedy, bool draft, int tm, int dm, const StatsLaunch& L)
{
    if (greedy) launch_rows_t<DT, true, false>(P, tm, dm, L);
    else if (draft) launch_rows_t<DT, false, true>(P, tm, dm, L);
    else launch_rows_t<DT, false, false>(P, tm, dm, L);
}

// `rows_max` bounds the target rows of one request and `drows_max` its draft
// rows; `rows_bound` bounds the rows of the whole pass (target and draft) and
// only sizes the flat grid.  P.plan must hold bs * (rows_max + drows_max)
// entries.
static void launch_stats(StatsParams P, int dt, bool a, int ddt, bool da, bool draft, bool greedy, int rows_max,
                         int drows_max, int64_t rows_bound, const RowSplit& sp, int32_t* gpre, const StatsLaunch& st)
{
    const int vec = dt == SPEC_F32 ? vec_of<SPEC_F32>() : vec_of<SPEC_BF16>();
    const int64_t cap = (int64_t)P.bs * (rows_max + drows_max);
    const bool flat = a && P.vocab % vec == 0 && (!draft || (ddt == dt && da)) && cap * sp.splits < INT32_MAX &&
                      (int64_t)P.bs * P.NR < INT32_MAX && P.n_rows <= INT32_MAX && P.dn_rows <= INT32_MAX;
    if (flat && rows_bound * 4 >= cap * 3 && P.bs <= 65535) {
        // the bound is close to every request's own: no row list
        if (dt == SPEC_F32) launch_rows_d<SPEC_F32>(P, greedy, draft, rows_max, drows_max, st);
        else launch_rows_d<SPEC_BF16>(P, greedy, draft, rows_max, drows_max, st);
        return;
    }
    if (flat) {
        const int64_t rows = rows_bound < cap ? (rows_bound > 0 ? rows_bound : 1) : cap;
        const int64_t grid = rows * sp.splits;
        if (dt == SPEC_F32) launch_flat_d<SPEC_F32>(P, greedy, draft, grid, st);
        else launch_flat_d<SPEC_BF16>(P, greedy, draft, grid, st);
        return;
    }
    // the other forms need no plan, but the residual bookkeeping still needs its reset
    if (P.done) hipLaunchKernelGGL(k_plan_rows<false>, dim3(1), dim3(kBlock), 0, st.st, P);
    const bool pipe = a && P.vocab % vec == 0 && P.bs <= kRowBaseLds && (int64_t)P.bs * rows_max <= kPipeMap;
    if (pipe) {
        const int64_t items = stats_items(P.bs, rows_max, sp);
        if (dt == SPEC_F32) {
            if (greedy) launch_pipe_d<SPEC_F32, true>(P, ddt, da, draft, false, items, st);
            else launch_pipe_d<SPEC_F32, false>(P, ddt, da, draft, false, items, st);
        } else {
            if (greedy) launch_pipe_d<SPEC_BF16, true>(P, ddt, da, draft, false, items, st);
            else launch_pipe_d<SPEC_BF16, false>(P, ddt, da, draft, false, items, st);
        }
        return;
    }
    const int64_t items = stats_items(P.bs, rows_max, sp);
    const bool gp = P.bs > kMaxLdsPrefix;
    if (gp) {
        P.gprefix = gpre;
        hipLaunchKernelGGL(k_plan, dim3(1), dim3(kBlock), 0, st.st, P, gpre);
    }
    if (greedy) {
        if (gp) launch_stats_g<true, true>(P, dt, a, ddt, da, draft, items, st);
        else launch_stats_g<true, false>(P, dt, a, ddt, da, draft, items, st);
    } else {
        if (gp) launch_stats_g<false, true>(P, dt, a, ddt, da, draft, items, st);
        else launch_stats_g<false, false>(P, dt, a, ddt, da, draft, items, st);
    }
}

}  // namespace spec

using namespace spec;

static int elem_bytes(int dt) { return dt == SPEC_F32 ? 4 : 2; }

// Row plan of the statistics pass: [rows] entries, then the count.
static size_t plan_bytes(int64_t rows) { return align256((size_t)rows * sizeof(int2)) + align256(sizeof(int32_t)); }

// Verify workspace: partials [bs, NR, splits] | row prefix [bs + 1] | row plan [bs * NR] |
// residual sums [bs, splits, kSubSums] | residual counters [2 bs]
size_t spec_verify_chain_ws(int32_t bs, int32_t vocab, int32_t ld, int32_t dtype)
{
    RowSplit sp = row_split(vocab, elem_bytes(dtype));
    const int NR = 2 * ld + 1;
    return align256((size_t)bs * NR * sp.splits * sizeof(Partial)) + align256((size_t)(bs + 1) * sizeof(int32_t)) +
           plan_bytes((int64_t)bs * NR) + align256((size_t)bs * sp.splits * kSubSums * sizeof(double)) +
           align256((size_t)2 * bs * sizeof(uint32_t));
}

// Tree verify workspace: partials [bs, rows_max, splits] | row prefix [bs + 1] | row plan [bs * rows_max]
size_t spec_verify_tree_ws(int32_t bs, int32_t vocab, int32_t rows_max, int32_t dtype)
{
    RowSplit sp = row_split(vocab, elem_bytes(dtype));
    return align256((size_t)bs * rows_max * sp.splits * sizeof(Partial)) +
           align256((size_t)(bs + 1) * sizeof(int32_t)) + plan_bytes((int64_t)bs * rows_max);
}

int spec_verify_chain_launch(const spec_verify_args* a, hipStream_t st)
{
    RowSplit sp = row_split(a->vocab, elem_bytes(a->dtype));
    const int NR = 2 * a->ld + 1;
    char* ws = (char*)a->workspace;
    ChainParams P;
    P.bs = a->bs; P.vocab = a->vocab; P.ld = a->ld;
    P.greedy = a->temperature == 0.0f;
    P.c = P.greedy ? 1.0f : kLog2e / a->temperature;
    P.logits = a->logits; P.dt = a->dtype; P.stride = a->row_stride; P.row_base = a->row_base;
    P.n_rows = a->n_logit_rows;
    P.dlogits = P.greedy ? nullptr : a->draft_logits; P.ddt = a->draft_dtype; P.dstride = a->draft_row_stride;
    P.drow_base = a->draft_row_base; P.dn_rows = a->n_draft_rows;
    P.tokens = a->tokens; P.slot_flags = a->slot_flags; P.n_slots = a->n_slots;
    P.u_acc = a->u_accept; P.u_smp = a->u_sample;
    P.rng = a->rng; P.rng_seed = a->rng_seed; P.rng_offset = a->rng_offset;
    P.accept_hist = a->out_accept_hist;
    P.out_tokens = a->out_tokens; P.out_num = a->out_num; P.out_acc = a->out_accepted;
    P.out_p = a->out_p; P.out_q = a->out_q; P.out_flags = a->out_flags; P.write_flags = a->write_flags;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len;
    P.ctx_len_out = a->ctx_len_out ? a->ctx_len_out : a->ctx_len; P.ctx_cap = a->ctx_cap;
    P.ng_draft = a->ctx ? a->ngram_draft : nullptr; P.ng_len = a->ngram_draft_len; P.ng_feat = a->ngram_feat;
    P.ng_min = a->ngram_n_min; P.ng_max = a->ngram_n_max; P.ng_ld = a->ngram_max_draft; P.ng_cap = a->ngram_copy_cap;
    P.wait_limit = a->residual_wait == 0 ? (1 << 20) : (a->residual_wait < 0 ? -1 : a->residual_wait);
    P.part = (Partial*)ws;
    ws += align256((size_t)a->bs * NR * sp.splits * sizeof(Partial));
    int32_t* gpre = (int32_t*)ws;
    ws += align256((size_t)(a->bs + 1) * sizeof(int32_t));
    int2* plan = (int2*)ws;
    int32_t* plan_count = (int32_t*)(ws + align256((size_t)a->bs * NR * sizeof(int2)));
    ws += plan_bytes((int64_t)a->bs * NR);
    P.sums = (double*)ws;
    ws += align256((size_t)a->bs * sp.splits * kSubSums * sizeof(double));
    P.done = (uint32_t*)ws;
    P.NR = NR; P.splits = sp.splits; P.chunk = sp.chunk;
    P.t_aligned = aligned16(a->logits, a->row_stride, a->dtype);
    P.d_aligned = P.dlogits && aligned16(a->draft_logits, a->draft_row_stride, a->draft_dtype);
    P.coal = P.t_aligned && P.d_aligned && a->dtype == a->draft_dtype &&
             a->vocab % (a->dtype == SPEC_F32 ? vec_of<SPEC_F32>() : vec_of<SPEC_BF16>()) == 0;

    const bool draft = !P.greedy && P.dlogits && a->slot_flags;
    StatsParams S;
    S.logits = a->logits; S.stride = a->row_stride; S.row_base = a->row_base; S.n_rows = a->n_logit_rows;
    S.dlogits = draft ? a->draft_logits : nullptr; S.dstride = a->draft_row_stride; S.drow_base = a->draft_row_base;
    S.dn_rows = a->n_draft_rows;
    S.counts = a->n_slots; S.cmin = 0; S.cmax = a->ld; S.cadd = 1;
    S.slot_flags = a->slot_flags; S.ld = a->ld;
    S.bs = a->bs; S.vocab = a->vocab; S.chunk = sp.chunk; S.splits = sp.splits; S.c = P.c;
    S.part = P.part; S.NR = NR; S.draft_base = a->ld + 1; S.gprefix = nullptr;
    S.plan = plan; S.plan_count = plan_count;
    S.done = draft ? P.done : nullptr; S.sums = P.sums;   // residual bookkeeping, reset by k_plan_rows
    // rows of the pass: b + 1 target rows per request and a draft row per slot
    const int64_t slots_all = (int64_t)a->bs * a->ld;
    const int64_t slots = a->max_slots > 0 && a->max_slots < slots_all ? a->max_slots : slots_all;
    const bool at = aligned16(a->logits, a->row_stride, a->dtype);
    const bool ad = draft && aligned16(a->draft_logits, a->draft_row_stride, a->draft_dtype);
    const StatsLaunch L{st, (hipEvent_t)a->prof_begin, (hipEvent_t)a->prof_end};
    launch_stats(S, a->dtype, at, a->draft_dtype, ad, draft, P.greedy, a->ld + 1, draft ? a->ld : 0,
                 a->bs + slots + (draft ? slots : 0), sp, gpre, L);
    const int tt = a->dtype, dd = P.dlogits ? a->draft_dtype : a->dtype;
    // residual chunks shared by K workgroups per request, about 5 each, and
    // no more than the chip holds at once for the batch: a workgroup that
    // starts after the others have taken every chunk still runs its whole
    // prologue, and the draw waits for its report
    const void* kern = (tt == SPEC_F32 && dd == SPEC_F32) ? (const void*)k_decide<SPEC_F32, SPEC_F32>
                     : (tt == SPEC_F32) ? (const void*)k_decide<SPEC_F32, SPEC_BF16>
                     : (dd == SPEC_F32) ? (const void*)k_decide<SPEC_BF16, SPEC_F32>
                                        : (const void*)k_decide<SPEC_BF16, SPEC_BF16>;
    int K = draft && P.coal && sp.splits <= kDBlock ? std::min(16, std::max(1, (sp.splits + 4) / 5)) : 1;
    if (K > 1) {
        const int64_t fit = (int64_t)blocks_per_cu(kern, kDBlock) * device_cus() / a->bs;
        K = (int)std::max<int64_t>(1, std::min<int64_t>(K, fit));
    }
    const dim3 g(a->bs, K), b(kDBlock);
    if (tt == SPEC_F32 && dd == SPEC_F32) hipLaunchKernelGGL((k_decide<SPEC_F32, SPEC_F32>), g, b, 0, st, P);
    else if (tt == SPEC_F32) hipLaunchKernelGGL((k_decide<SPEC_F32, SPEC_BF16>), g, b, 0, st, P);
    else if (dd == SPEC_F32) hipLaunchKernelGGL((k_decide<SPEC_BF16, SPEC_F32>), g, b, 0, st, P);
    else hipLaunchKernelGGL((k_decide<SPEC_BF16, SPEC_BF16>), g, b, 0, st, P);
    return spec_record_hip_error(hipGetLastError());
}

int spec_verify_tree_launch(const spec_tree_verify_args* a, hipStream_t st)
{
    RowSplit sp = row_split(a->vocab, elem_bytes(a->dtype));
    char* ws = (char*)a->workspace;
    TreeParams P;
    P.bs = a->bs; P.vocab = a->vocab; P.rows_max = a->rows_max;
    P.node_token = a->node_token; P.parent_row = a->parent_row; P.n_rows = a->n_rows;
    P.out_tokens = a->out_tokens; P.out_num = a->out_num; P.out_path = a->out_path_rows; P.out_argmax = a->out_argmax;
    P.out_flags = a->out_flags;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len;
    P.ctx_len_out = a->ctx_len_out ? a->ctx_len_out : a->ctx_len; P.ctx_cap = a->ctx_cap;
    P.part = (Partial*)ws;
    P.splits = sp.splits;
    int32_t* gpre = (int32_t*)(ws + align256((size_t)a->bs * a->rows_max * sp.splits * sizeof(Partial)));
    int2* plan = (int2*)((char*)gpre + align256((size_t)(a->bs + 1) * sizeof(int32_t)));
    int32_t* plan_count = (int32_t*)((char*)plan + align256((size_t)a->bs * a->rows_max * sizeof(int2)));
    StatsParams S;
    S.logits = a->logits; S.stride = a->row_stride; S.row_base = a->row_base; S.n_rows = a->n_logit_rows;
    S.dlogits = nullptr; S.dstride = 0; S.drow_base = nullptr; S.dn_rows = 0;
    S.counts = a->n_rows; S.cmin = 1; S.cmax = a->rows_max; S.cadd = 0;
    S.slot_flags = nullptr; S.ld = 0;
    S.bs = a->bs; S.vocab = a->vocab; S.chunk = sp.chunk; S.splits = sp.splits; S.c = 1.0f;
    S.part = P.part; S.NR = a->rows_max; S.draft_base = 0; S.gprefix = nullptr;
    S.plan = plan; S.plan_count = plan_count;
    S.done = nullptr; S.sums = nullptr;
    const StatsLaunch L{st, (hipEvent_t)a->prof_begin, (hipEvent_t)a->prof_end};
    launch_stats(S, a->dtype, aligned16(a->logits, a->row_stride, a->dtype), SPEC_F32, false, false, true,
                 a->rows_max, 0, (int64_t)a->bs * a->rows_max, sp, gpre, L);
    if ((int64_t)P.rows_max * P.splits <= 16 * kWave)
        hipLaunchKernelGGL(k_tree_walk<16>, dim3(a->bs), dim3(kWave), 0, st, P);
    else
        hipLaunchKernelGGL(k_tree_walk<32>, dim3(a->bs), dim3(kWave), 0, st, P);
    return spec_record_hip_error(hipGetLastError());
}

// ---------------------------------------------------------------------------
// the chain verifier without a caller workspace
// ---------------------------------------------------------------------------

// Scratch of spec_verify_chain_noalloc: one array per device, held from the
// library's first use on the device until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host the name is a stand-in,
// not a device address): it uses the device address looked up once per
// device below.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

static std::atomic<void*> g_scratch_ptr[64];

// Device address of `scratch` on the current device: hipGetSymbolAddress on
// the first call on a device (with that device current), then the kept value.
static int scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return spec_record_hip_error(e);
    if (dev < 0 || dev >= 64) return SPEC_EINVAL;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_cache_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return spec_record_hip_error(e);
            if (!p) return spec_record_hip_error(hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SPEC_OK;
}

// The scratch the verifier needs (partials, row prefix and plan, residual
// sums and counters) comes from the device array; every part that must start
// at a known value is set by the call's own kernels (the statistics pass
// resets the residual counters and sums), so nothing is cleared here.
int spec_verify_chain_noalloc_launch(const spec_verify_args* a, hipStream_t st)
{
    const size_t need = spec_verify_chain_ws(a->bs, a->vocab, a->ld, a->dtype);
    if (need > (size_t)SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_EWORKSPACE;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != SPEC_OK) return rc;
    spec_verify_args b = *a;
    b.workspace = ws;
    b.workspace_bytes = (size_t)SPEC_NOALLOC_SCRATCH_BYTES;
    return spec_verify_chain_launch(&b, st);
}
