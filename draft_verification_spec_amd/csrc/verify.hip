// Chain and tree verification kernels.
//
// Chain rule: speculative sampling as in the LongSpark page ("Efficient
// speculative decoding with a fixed-cost parallel drafter", Section 2.1) --
// accept y_i with probability min(1, p_i(y_i)/q_i(y_i)); at the first reject
// draw from norm(max(0, p_i - q_i)); after the last slot draw the bonus from
// p_{b+1}.  Point-mass slots (Hybrid Spark, Section 5.8 and Appendix H) use
// q = delta_y.  At T = 0 a draft is accepted iff it is the target argmax
// (Hybrid Spark, Appendix H; AdaSpark, Section 2.2).
//
// Data flow (one stream, no host synchronisation):
//   k_row_stats   : every read logit row is cut into chunks; one workgroup per
//                   (chunk, request) streams the request's rows through that
//                   chunk with 16-byte loads and keeps an online (max, sum of
//                   2^(z*c - max*c)) per thread, c = log2(e)/T; at T = 0 a
//                   (max, first argmax) pair instead.  Partials go to the
//                   workspace.  This is the HBM-bound pass.
//   k_decide      : one workgroup per request merges the chunk partials of its
//                   rows, evaluates p(y), q(y) for every slot in parallel,
//                   finds the first rejection and records what to sample.
//   k_sample_part : chunk sums (fp64) of the residual / bonus weights.
//   k_sample_final: finds the chunk holding u*W, rescans it tile by tile with a
//                   workgroup prefix sum, writes the token, commits.
#include "common.hpp"

namespace spec {

constexpr int kBlock = 256;

struct Dec {
    int32_t mode;   // 0: nothing to draw; 1: from p of row_t; 2: max(0, p - q); 3: p without y
    int32_t nacc;
    int32_t y;
    float Ot, Od;   // base-2 offsets of the target / draft rows
    float pad0;
    int64_t row_t, row_d;
    double Zt, Zd;  // base-2 normalisers relative to the offsets
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t e)
{
    if constexpr (DT == SPEC_F32) {
        return ((const float*)base)[e];
    } else {
        return bf16_bits_to_float(((const uint16_t*)base)[e]);
    }
}

template <int DT, int VEC>
__device__ __forceinline__ void loadv(const void* base, int64_t e, float* v)
{
    if constexpr (VEC == 1) {
        v[0] = load1<DT>(base, e);
    } else if constexpr (DT == SPEC_F32) {
        static_assert(VEC == 4, "fp32 vectors are 16 bytes");
        float4 x = *(const float4*)((const float*)base + e);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else if constexpr (VEC == 8) {
        uint4 x = *(const uint4*)((const uint16_t*)base + e);
        v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
        v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
        v[4] = __uint_as_float(x.z << 16); v[5] = __uint_as_float(x.z & 0xFFFF0000u);
        v[6] = __uint_as_float(x.w << 16); v[7] = __uint_as_float(x.w & 0xFFFF0000u);
    } else {
        static_assert(VEC == 4, "bf16 vectors are 8 or 16 bytes");
        uint2 x = *(const uint2*)((const uint16_t*)base + e);
        v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
        v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
    }
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const void* base, int64_t row, int64_t stride)
{
    return (const char*)base + row * stride * (DT == SPEC_F32 ? 4 : 2);
}

// ---------------------------------------------------------------------------
// online softmax statistics
// ---------------------------------------------------------------------------

// (m, s): m = largest raw logit seen, s = sum of 2^(z*c - m*c) (the offset m*c
// is always recomputed the same way, so rescaling stays consistent).
template <int N>
__device__ __forceinline__ void sm_update(const float* v, float c, float& m, float& s)
{
    float tm = v[0];
#pragma unroll
    for (int i = 1; i < N; ++i) tm = fmaxf(tm, v[i]);
    if (tm > m) {
        float on = tm * c;
        s = (m == -INFINITY) ? 0.0f : s * fast_exp2(m * c - on);
        m = tm;
    }
    if (m != -INFINITY) {
        const float o = m * c;
#pragma unroll
        for (int i = 0; i < N; ++i) s += fast_exp2(fmaf(v[i], c, -o));
    } else if (tm != tm) {
        s = __builtin_nanf("");  // a tile of NaN before any finite value
    }
}

__device__ __forceinline__ void sm_combine(float& m, float& s, float m2, float s2, float c)
{
    if (m2 > m) {
        float t = m; m = m2; m2 = t;
        t = s; s = s2; s2 = t;
    }
    if (m2 == -INFINITY) {
        if (s2 != s2) s = s2;
        return;
    }
    s = s + s2 * fast_exp2(m2 * c - m * c);
}

// (best, idx, bad): largest logit, its lowest index, any NaN/+Inf seen.
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

template <int DT, int VEC, int U>
__device__ __forceinline__ void chunk_softmax(const void* row, int64_t lo, int64_t hi, float c, float& m, float& s)
{
    const int64_t hv = lo + (hi - lo) / VEC * VEC;
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    int64_t e = lo + (int64_t)threadIdx.x * VEC;
    for (; e + (U - 1) * STEP < hv; e += U * STEP) {
        float v[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) loadv<DT, VEC>(row, e + u * STEP, v + u * VEC);
        sm_update<U * VEC>(v, c, m, s);
    }
    for (; e < hv; e += STEP) {
        float v[VEC];
        loadv<DT, VEC>(row, e, v);
        sm_update<VEC>(v, c, m, s);
    }
    for (int64_t t = hv + threadIdx.x; t < hi; t += kBlock) {
        float v = load1<DT>(row, t);
        sm_update<1>(&v, c, m, s);
    }
}

template <int DT, int VEC, int U>
__device__ __forceinline__ void chunk_argmax(const void* row, int64_t lo, int64_t hi, ArgAcc& a)
{
    const int64_t hv = lo + (hi - lo) / VEC * VEC;
    constexpr int64_t STEP = (int64_t)kBlock * VEC;
    int64_t e = lo + (int64_t)threadIdx.x * VEC;
    for (; e + (U - 1) * STEP < hv; e += U * STEP) {
        float v[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) loadv<DT, VEC>(row, e + u * STEP, v + u * VEC);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < VEC; ++k) am_update(v[u * VEC + k], (int32_t)(e + u * STEP + k), a);
    }
    for (; e < hv; e += STEP) {
        float v[VEC];
        loadv<DT, VEC>(row, e, v);
#pragma unroll
        for (int k = 0; k < VEC; ++k) am_update(v[k], (int32_t)(e + k), a);
    }
    for (int64_t t = hv + threadIdx.x; t < hi; t += kBlock) am_update(load1<DT>(row, t), (int32_t)t, a);
}

// Partial of one (row, chunk): T > 0 -> (m, s); T = 0 -> (best, idx bits | bad in sign of a NaN).
struct Partial {
    float a;
    float b;
};

// Row set of a request: rows row_base[r] + k, k < count, count from a device
// array clamped to [cmin, cmax] plus cadd.  A draft pass skips point-mass slots.
struct RowSet {
    const void* logits;
    int64_t stride;
    const int64_t* row_base;
    int64_t n_rows;          // rows in the logits buffer (bounds)
    const int32_t* counts;
    int32_t cmin, cmax, cadd;
    const uint8_t* skip_pm;  // slot flags [bs, ld] or null
    int32_t ld;
    int32_t slot_base;       // partial row index offset
};

template <int DT, int VEC, bool GREEDY>
__global__ __launch_bounds__(kBlock) void k_row_stats(RowSet rs, int32_t vocab, int64_t chunk, int32_t splits,
                                                      float c, Partial* __restrict__ part, int32_t NR)
{
    const int s = blockIdx.x;
    const int r = blockIdx.y;
    int cnt = rs.counts[r];
    cnt = (cnt < rs.cmin ? rs.cmin : (cnt > rs.cmax ? rs.cmax : cnt)) + rs.cadd;
    const int64_t lo = (int64_t)s * chunk;
    const int64_t hi = (lo + chunk < vocab) ? lo + chunk : vocab;
    const int64_t base = rs.row_base[r];
    __shared__ float sh_a[kBlock / kWave];
    __shared__ float sh_b[kBlock / kWave];
    __shared__ int32_t sh_i[kBlock / kWave];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    for (int k = 0; k < cnt; ++k) {
        if (rs.skip_pm && (rs.skip_pm[(int64_t)r * rs.ld + k] & SPEC_SLOT_POINT_MASS)) continue;
        Partial* out = part + ((int64_t)r * NR + rs.slot_base + k) * splits + s;
        const int64_t row = base + k;
        if (row < 0 || row >= rs.n_rows) {
            if (threadIdx.x == 0) { out->a = __builtin_nanf(""); out->b = __builtin_nanf(""); }
            continue;
        }
        const void* rp = row_ptr<DT>(rs.logits, row, rs.stride);
        if constexpr (!GREEDY) {
            float m = -INFINITY, sum = 0.0f;
            chunk_softmax<DT, VEC, 2>(rp, lo, hi, c, m, sum);
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(sum, o, kWave);
                sm_combine(m, sum, m2, s2, c);
            }
            if (lane == 0) { sh_a[wid] = m; sh_b[wid] = sum; }
            __syncthreads();
            if (threadIdx.x == 0) {
                for (int w = 1; w < kBlock / kWave; ++w) sm_combine(m, sum, sh_a[w], sh_b[w], c);
                out->a = m;
                out->b = sum;
            }
            __syncthreads();
        } else {
            ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
            chunk_argmax<DT, VEC, 2>(rp, lo, hi, acc);
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                ArgAcc b{__shfl_xor(acc.best, o, kWave), __shfl_xor(acc.idx, o, kWave), __shfl_xor(acc.bad, o, kWave)};
                am_combine(acc, b);
            }
            if (lane == 0) { sh_a[wid] = acc.best; sh_i[wid] = acc.idx | (acc.bad ? (int32_t)0x80000000 : 0); }
            __syncthreads();
            if (threadIdx.x == 0) {
                acc.bad = 0;
                for (int w = 0; w < kBlock / kWave; ++w) {
                    ArgAcc b{sh_a[w], sh_i[w] & 0x7FFFFFFF, (sh_i[w] >> 31) & 1};
                    am_combine(acc, b);
                }
                out->a = acc.best;
                out->b = __int_as_float(acc.idx | (acc.bad ? (int32_t)0x80000000 : 0));
            }
            __syncthreads();
        }
    }
}

// Merge the chunk partials of one row.  Softmax: returns false when the row
// is unusable; *O = m*c, *Z = sum relative to O (fp64).
__device__ bool merge_softmax(const Partial* p, int splits, float c, float* O, double* Z)
{
    float m = -INFINITY;
    bool nan = false;
    for (int s = 0; s < splits; ++s) {
        m = fmaxf(m, p[s].a);
        nan |= (p[s].a != p[s].a) || (p[s].b != p[s].b);
    }
    const float o = m * c;
    double z = 0.0;
    for (int s = 0; s < splits; ++s) {
        if (p[s].a == -INFINITY) continue;
        z += (double)p[s].b * (double)fast_exp2(p[s].a * c - o);
    }
    *O = o;
    *Z = z;
    return !nan && m != -INFINITY && m != INFINITY && z > 0.0 && z < INFINITY;
}

__device__ bool merge_argmax(const Partial* p, int splits, int32_t* idx)
{
    ArgAcc acc{-INFINITY, 0x7FFFFFFF, 0};
    for (int s = 0; s < splits; ++s) {
        int32_t bits = __float_as_int(p[s].b);
        ArgAcc b{p[s].a, bits & 0x7FFFFFFF, (bits >> 31) & 1};
        if (p[s].a != p[s].a) b.bad = 1;
        am_combine(acc, b);
    }
    *idx = acc.idx;
    return !acc.bad && acc.idx != 0x7FFFFFFF;
}

// ---------------------------------------------------------------------------
// decide
// ---------------------------------------------------------------------------

struct ChainParams {
    int32_t bs, vocab, ld;
    float c;            // log2(e) / T (T > 0)
    int32_t greedy;
    const void* logits; int32_t dt; int64_t stride; const int64_t* row_base; int64_t n_rows;
    const void* dlogits; int32_t ddt; int64_t dstride; const int64_t* drow_base; int64_t dn_rows;
    const int32_t* tokens; const uint8_t* slot_flags; const int32_t* n_slots;
    const float* u_acc; const float* u_smp;
    int32_t* out_tokens; int32_t* out_num; int32_t* out_acc; float* out_p; float* out_q; uint32_t* out_flags;
    int32_t* ctx; int64_t ctx_stride; int32_t* ctx_len; int32_t ctx_cap;
    Partial* part; int32_t NR; int32_t splits; int64_t chunk;
    Dec* dec; double* sums;
};

__device__ __forceinline__ float logit_at(const void* base, int dt, int64_t row, int64_t stride, int64_t v)
{
    return dt == SPEC_F32 ? ((const float*)base)[row * stride + v]
                          : bf16_bits_to_float(((const uint16_t*)base)[row * stride + v]);
}

constexpr int kDecideBlock = 128;  // >= 2 * SPEC_MAX_DRAFT + 1 rows

__global__ __launch_bounds__(kDecideBlock) void k_decide(ChainParams P)
{
    const int r = blockIdx.x;
    const int t = threadIdx.x;
    const int ld = P.ld;
    int b = P.n_slots[r];
    const bool badlen = (b < 0 || b > ld);
    b = b < 0 ? 0 : (b > ld ? ld : b);
    __shared__ float sO[kDecideBlock];
    __shared__ double sZ[kDecideBlock];
    __shared__ int32_t sArg[kDecideBlock];
    __shared__ int32_t sOk[kDecideBlock];
    __shared__ uint32_t sFlags;
    __shared__ uint64_t sRej;
    if (t == 0) { sFlags = badlen ? SPEC_FLAG_BAD_LENGTH : 0u; sRej = 0; }
    // row t: target rows 0..b, draft rows ld+1 .. ld+b (probabilistic slots, T > 0)
    bool is_row = false;
    if (t <= b) is_row = true;
    else if (!P.greedy && P.dlogits && t >= ld + 1 && t <= ld + b) {
        const int i = t - ld - 1;
        is_row = !(P.slot_flags && (P.slot_flags[(int64_t)r * ld + i] & SPEC_SLOT_POINT_MASS));
    }
    sOk[t] = 0;
    if (is_row) {
        const Partial* p = P.part + ((int64_t)r * P.NR + t) * P.splits;
        if (P.greedy) {
            int32_t idx;
            sOk[t] = merge_argmax(p, P.splits, &idx);
            sArg[t] = idx;
        } else {
            float O; double Z;
            sOk[t] = merge_softmax(p, P.splits, P.c, &O, &Z);
            sO[t] = O;
            sZ[t] = Z;
        }
    }
    __syncthreads();
    // slot i = t < b: p(y), q(y), accept
    bool acc = true;
    uint32_t fl = 0;
    if (t < b) {
        const int64_t off = (int64_t)r * ld + t;
        const int32_t y = P.tokens[off];
        const bool pm = !P.slot_flags || (P.slot_flags[off] & SPEC_SLOT_POINT_MASS);
        const bool bad = (y < 0 || y >= P.vocab);
        if (bad) fl |= SPEC_FLAG_BAD_TOKEN;
        const int64_t trow = P.row_base[r] + t;
        if (!sOk[t]) fl |= SPEC_FLAG_BAD_LOGITS;
        double p = 0.0, q = 1.0;
        if (P.greedy) {
            p = (!bad && sOk[t] && sArg[t] == y) ? 1.0 : 0.0;
            acc = (p == 1.0);
        } else {
            if (!bad && sOk[t]) {
                float z = logit_at(P.logits, P.dt, trow, P.stride, y);
                p = (double)fast_exp2(fmaf(z, P.c, -sO[t])) / sZ[t];
            }
            if (!pm) {
                const int dr = ld + 1 + t;
                if (!sOk[dr]) fl |= SPEC_FLAG_BAD_LOGITS;
                q = 0.0;
                if (!bad && sOk[dr] && P.dlogits) {
                    const int64_t drow = P.drow_base[r] + t;
                    float w = logit_at(P.dlogits, P.ddt, drow, P.dstride, y);
                    q = (double)fast_exp2(fmaf(w, P.c, -sO[dr])) / sZ[dr];
                }
            }
            const double rho = q > 0.0 ? p / q : 0.0;
            acc = (double)P.u_acc[off] < rho;
        }
        if (P.out_p) P.out_p[off] = (float)p;
        if (P.out_q) P.out_q[off] = (float)q;
        if (!acc) atomicOr((unsigned long long*)&sRej, 1ull << t);
        if (fl) atomicOr(&sFlags, fl);
    } else if (t < ld) {
        const int64_t off = (int64_t)r * ld + t;
        if (P.out_p) P.out_p[off] = 0.0f;
        if (P.out_q) P.out_q[off] = 0.0f;
    }
    __syncthreads();
    const uint64_t rej = sRej;
    const int nacc = rej ? (int)__builtin_ctzll(rej) : b;
    // outputs: accepted prefix, -1 padding
    for (int i = t; i <= ld; i += kDecideBlock)
        P.out_tokens[(int64_t)r * (ld + 1) + i] = (i < nacc) ? P.tokens[(int64_t)r * ld + i] : -1;
    if (t == 0) {
        uint32_t flags = sFlags;
        if (nacc == b && !sOk[b]) flags |= SPEC_FLAG_BAD_LOGITS;
        P.out_num[r] = nacc + 1;
        P.out_acc[r] = nacc;
        Dec d;
        d.nacc = nacc;
        d.mode = 0;
        d.y = -1;
        d.Ot = d.Od = 0.0f;
        d.pad0 = 0.0f;
        d.row_t = P.row_base[r] + nacc;
        d.row_d = -1;
        d.Zt = d.Zd = 1.0;
        if (P.greedy) {
            int32_t tok = sOk[nacc] ? sArg[nacc] : -1;
            if (tok == 0x7FFFFFFF) tok = -1;
            P.out_tokens[(int64_t)r * (ld + 1) + nacc] = tok;
        } else if (!(d.row_t >= 0 && d.row_t < P.n_rows) || !sOk[nacc]) {
            d.mode = 0;          // unusable row: the token stays -1, flagged above
            flags |= SPEC_FLAG_BAD_LOGITS;
        } else {
            d.Ot = sO[nacc];
            d.Zt = sZ[nacc];
            if (nacc == b) {
                d.mode = 1;
            } else {
                const int64_t off = (int64_t)r * ld + nacc;
                const int32_t y = P.tokens[off];
                const bool pm = !P.slot_flags || (P.slot_flags[off] & SPEC_SLOT_POINT_MASS);
                const bool bad = (y < 0 || y >= P.vocab);
                const int dr = ld + 1 + nacc;
                if (bad) {
                    d.mode = 1;
                } else if (pm) {
                    d.mode = 3;
                    d.y = y;
                } else if (sOk[dr] && P.dlogits) {
                    d.mode = 2;
                    d.y = y;
                    d.row_d = P.drow_base[r] + nacc;
                    d.Od = sO[dr];
                    d.Zd = sZ[dr];
                } else {
                    d.mode = 1;  // unusable draft row (flagged): fall back to p
                }
            }
        }
        P.dec[r] = d;
        if (flags) atomicOr(&P.out_flags[r], flags);
    }
}

// ---------------------------------------------------------------------------
// sampling
// ---------------------------------------------------------------------------

// Weight of token v (fp64) for the draw described by d.
template <int DTT, int DTD>
__device__ __forceinline__ double draw_weight(const ChainParams& P, const Dec& d, int mode, double ratio, int64_t v)
{
    const float z = logit_at(P.logits, DTT, d.row_t, P.stride, v);
    const double ep = (double)fast_exp2(fmaf(z, P.c, -d.Ot));
    if (mode == 1) return ep;
    if (mode == 3) return v == d.y ? 0.0 : ep;
    const float w = logit_at(P.dlogits, DTD, d.row_d, P.dstride, v);
    const double eq = (double)fast_exp2(fmaf(w, P.c, -d.Od));
    const double x = ep - eq * ratio;
    return x > 0.0 ? x : 0.0;
}

__device__ double block_sum_f64(double v)
{
    __shared__ double sh[kBlock / kWave];
    v = wave_sum(v);
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < kBlock / kWave; ++w) tot += sh[w];
    return tot;
}

// Exclusive prefix sum over the workgroup (thread order); also returns the total.
__device__ double block_exclusive_f64(double v, double* total)
{
    __shared__ double sh[kBlock / kWave];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    double inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double u = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += u;
    }
    __syncthreads();
    if (lane == kWave - 1) sh[wid] = inc;
    __syncthreads();
    double before = 0.0, tot = 0.0;
    for (int w = 0; w < kBlock / kWave; ++w) {
        if (w < wid) before += sh[w];
        tot += sh[w];
    }
    *total = tot;
    return before + inc - v;
}

template <int DTT, int DTD>
__global__ __launch_bounds__(kBlock) void k_sample_partial(ChainParams P)
{
    const int s = blockIdx.x, r = blockIdx.y;
    const Dec d = P.dec[r];
    if (d.mode == 0) return;
    const int64_t lo = (int64_t)s * P.chunk;
    const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
    const double ratio = d.Zt / d.Zd;
    double acc = 0.0;
    for (int64_t v = lo + threadIdx.x; v < hi; v += kBlock) acc += draw_weight<DTT, DTD>(P, d, d.mode, ratio, v);
    const double tot = block_sum_f64(acc);
    if (threadIdx.x == 0) P.sums[(int64_t)r * P.splits + s] = tot;
}

// Search [lo, hi) for the first token whose running weight exceeds t, tile by
// tile in index order.  Returns -1 when rounding left t past the range.
template <int DTT, int DTD>
__device__ int64_t search_range(const ChainParams& P, const Dec& d, int mode, double ratio, int64_t lo, int64_t hi,
                                double t, int64_t* last_pos)
{
    // Tile by tile in index order: each thread holds E consecutive weights, a
    // workgroup exclusive scan gives its running start; the lowest position
    // whose running sum passes t wins (atomicMin keeps the choice unique when
    // rounding lets two neighbours both claim it).
    __shared__ unsigned long long sh_found;
    __shared__ double sh_base;
    __shared__ unsigned long long sh_lp;
    if (threadIdx.x == 0) { sh_found = ~0ull; sh_base = 0.0; sh_lp = 0ull; }
    int64_t lp = -1;
    __syncthreads();
    constexpr int E = 4;
    for (int64_t tile = lo; tile < hi; tile += (int64_t)kBlock * E) {
        const int64_t a = tile + (int64_t)threadIdx.x * E;
        double w[E];
        double mine = 0.0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            w[k] = (a + k < hi) ? draw_weight<DTT, DTD>(P, d, mode, ratio, a + k) : 0.0;
            mine += w[k];
            if (w[k] > 0.0) lp = a + k;
        }
        double total;
        const double ex = block_exclusive_f64(mine, &total);
        const double base = sh_base;
        double c = base + ex;
        if (c + mine > t) {
            int64_t pos = -1, lastpos = -1;
            for (int k = 0; k < E; ++k) {
                if (w[k] > 0.0) {
                    lastpos = a + k;
                    if (pos < 0 && c + w[k] > t) pos = a + k;
                }
                c += w[k];
            }
            if (pos < 0) pos = lastpos;
            if (pos >= 0) atomicMin(&sh_found, (unsigned long long)pos);
        }
        __syncthreads();
        if (threadIdx.x == 0) sh_base = base + total;
        __syncthreads();
        if (sh_found != ~0ull) break;
    }
    if (lp >= 0) atomicMax(&sh_lp, (unsigned long long)(lp + 1));
    __syncthreads();
    *last_pos = (int64_t)sh_lp - 1;
    return sh_found == ~0ull ? -1 : (int64_t)sh_found;
}

template <int DTT, int DTD>
__global__ __launch_bounds__(kBlock) void k_sample_final(ChainParams P)
{
    const int r = blockIdx.x;
    const Dec d = P.dec[r];
    const int ld = P.ld;
    __shared__ int32_t sh_tok;
    __shared__ uint32_t sh_fl;
    if (threadIdx.x == 0) { sh_tok = -1; sh_fl = 0; }
    __syncthreads();
    if (d.mode != 0) {
        // locate the chunk
        __shared__ int32_t sh_chunk;
        __shared__ double sh_t, sh_W;
        if (threadIdx.x == 0) {
            double W = 0.0;
            for (int s = 0; s < P.splits; ++s) W += P.sums[(int64_t)r * P.splits + s];
            sh_W = W;
            const double t = (double)P.u_smp[r] * W;
            double cum = 0.0;
            int sc = P.splits - 1;
            for (int s = 0; s < P.splits; ++s) {
                const double x = P.sums[(int64_t)r * P.splits + s];
                if (cum + x > t) { sc = s; break; }
                cum += x;
            }
            sh_chunk = sc;
            sh_t = t - cum;
        }
        __syncthreads();
        const double ratio = d.Zt / d.Zd;
        int64_t lastp = -1, found = -1;
        if (sh_W > 0.0 && sh_W < INFINITY) {
            const int64_t lo = (int64_t)sh_chunk * P.chunk;
            const int64_t hi = (lo + P.chunk < P.vocab) ? lo + P.chunk : P.vocab;
            found = search_range<DTT, DTD>(P, d, d.mode, ratio, lo, hi, sh_t, &lastp);
        } else {
            // the residual had no mass (not reachable in exact arithmetic): draw from p
            if (threadIdx.x == 0) sh_fl |= SPEC_FLAG_RESIDUAL_ZERO;
            double acc = 0.0;
            for (int64_t v = threadIdx.x; v < P.vocab; v += kBlock) acc += draw_weight<DTT, DTD>(P, d, 1, ratio, v);
            const double W1 = block_sum_f64(acc);
            found = search_range<DTT, DTD>(P, d, 1, ratio, 0, P.vocab, (double)P.u_smp[r] * W1, &lastp);
        }
        if (threadIdx.x == 0) sh_tok = (int32_t)(found >= 0 ? found : lastp);
        __syncthreads();
        if (threadIdx.x == 0) P.out_tokens[(int64_t)r * (ld + 1) + d.nacc] = sh_tok;
    }
    // commit
    if (P.ctx) {
        __shared__ int32_t sh_len, sh_n, sh_ok;
        if (threadIdx.x == 0) {
            sh_len = P.ctx_len[r];
            sh_n = P.out_num[r];
            sh_ok = (sh_len >= 0 && sh_len + sh_n <= P.ctx_cap);
            if (!sh_ok) sh_fl |= SPEC_FLAG_CTX_OVERFLOW;
        }
        __syncthreads();
        if (sh_ok) {
            for (int i = threadIdx.x; i < sh_n; i += kBlock) {
                int32_t tok = (d.mode != 0 && i == d.nacc) ? sh_tok : P.out_tokens[(int64_t)r * (ld + 1) + i];
                P.ctx[(int64_t)r * P.ctx_stride + sh_len + i] = tok;
            }
            __syncthreads();
            if (threadIdx.x == 0) P.ctx_len[r] = sh_len + sh_n;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0 && sh_fl) atomicOr(&P.out_flags[r], sh_fl);
}

// ---------------------------------------------------------------------------
// tree walk (greedy)
// ---------------------------------------------------------------------------

struct TreeParams {
    int32_t bs, vocab, rows_max;
    const int64_t* row_base; int64_t n_rows_buf;
    const int32_t* node_token; const int32_t* parent_row; const int32_t* n_rows;
    int32_t* out_tokens; int32_t* out_num; int32_t* out_path; int32_t* out_argmax; uint32_t* out_flags;
    int32_t* ctx; int64_t ctx_stride; int32_t* ctx_len; int32_t ctx_cap;
    Partial* part; int32_t splits;
};

__global__ __launch_bounds__(kWave) void k_tree_walk(TreeParams P)
{
    const int r = blockIdx.x, t = threadIdx.x;
    const int rm = P.rows_max;
    int n = P.n_rows[r];
    const bool badlen = (n < 1 || n > rm);
    n = n < 1 ? 1 : (n > rm ? rm : n);
    __shared__ int32_t sArg[SPEC_MAX_ROWS];
    __shared__ int32_t sOk[SPEC_MAX_ROWS];
    __shared__ int32_t sTok[SPEC_MAX_ROWS];
    __shared__ int32_t sPar[SPEC_MAX_ROWS];
    __shared__ int32_t sOut[SPEC_MAX_ROWS];
    __shared__ int32_t sPath[SPEC_MAX_ROWS];
    __shared__ int32_t sNum;
    __shared__ uint32_t sFl;
    if (t < n) {
        int32_t idx;
        sOk[t] = merge_argmax(P.part + ((int64_t)r * rm + t) * P.splits, P.splits, &idx);
        sArg[t] = (idx == 0x7FFFFFFF) ? -1 : idx;
        sTok[t] = P.node_token[(int64_t)r * rm + t];
        sPar[t] = P.parent_row[(int64_t)r * rm + t];
    }
    for (int i = t; i < rm; i += kWave) { sOut[i] = -1; sPath[i] = -1; }
    __syncthreads();
    if (t == 0) {
        uint32_t fl = badlen ? SPEC_FLAG_BAD_LENGTH : 0u;
        for (int i = 0; i < n; ++i) if (!sOk[i]) fl |= SPEC_FLAG_BAD_LOGITS;
        int u = 0, k = 0;
        sPath[0] = 0;
        for (;;) {
            const int a = sArg[u];
            int next = -1;
            for (int c = 1; c < n; ++c)
                if (sPar[c] == u && sTok[c] == a) { next = c; break; }
            sOut[k++] = a;
            if (next < 0 || k >= rm) break;
            u = next;
            sPath[k] = u;
        }
        sNum = k;
        sFl = fl;
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
        if (t == 0 && ok) P.ctx_len[r] = len + sNum;
    }
    if (t == 0 && fl) atomicOr(&P.out_flags[r], fl);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

template <bool GREEDY>
static void launch_stats(int dt, bool aligned, RowSet rs, int vocab, RowSplit sp, int bs, float c, Partial* part,
                         int NR, hipStream_t st)
{
    dim3 grid(sp.splits, bs);
    if (dt == SPEC_F32) {
        if (aligned) hipLaunchKernelGGL((k_row_stats<SPEC_F32, 4, GREEDY>), grid, dim3(kBlock), 0, st, rs, vocab, sp.chunk, sp.splits, c, part, NR);
        else hipLaunchKernelGGL((k_row_stats<SPEC_F32, 1, GREEDY>), grid, dim3(kBlock), 0, st, rs, vocab, sp.chunk, sp.splits, c, part, NR);
    } else {
        if (aligned) hipLaunchKernelGGL((k_row_stats<SPEC_BF16, 8, GREEDY>), grid, dim3(kBlock), 0, st, rs, vocab, sp.chunk, sp.splits, c, part, NR);
        else hipLaunchKernelGGL((k_row_stats<SPEC_BF16, 1, GREEDY>), grid, dim3(kBlock), 0, st, rs, vocab, sp.chunk, sp.splits, c, part, NR);
    }
}

static bool aligned16(const void* p, int64_t stride, int dt)
{
    const int64_t es = dt == SPEC_F32 ? 4 : 2;
    return ((uintptr_t)p % 16 == 0) && ((stride * es) % 16 == 0);
}

}  // namespace spec

using namespace spec;

size_t spec_verify_chain_ws(int32_t bs, int32_t vocab, int32_t ld)
{
    RowSplit sp = row_split(bs, vocab);
    const int NR = 2 * ld + 1;
    return align256((size_t)bs * NR * sp.splits * sizeof(Partial)) + align256((size_t)bs * sizeof(Dec)) +
           align256((size_t)bs * sp.splits * sizeof(double));
}

size_t spec_verify_tree_ws(int32_t bs, int32_t vocab, int32_t rows_max)
{
    RowSplit sp = row_split(bs, vocab);
    return align256((size_t)bs * rows_max * sp.splits * sizeof(Partial));
}

int spec_verify_chain_launch(const spec_verify_args* a, hipStream_t st)
{
    RowSplit sp = row_split(a->bs, a->vocab);
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
    P.out_tokens = a->out_tokens; P.out_num = a->out_num; P.out_acc = a->out_accepted;
    P.out_p = a->out_p; P.out_q = a->out_q; P.out_flags = a->out_flags;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len; P.ctx_cap = a->ctx_cap;
    P.part = (Partial*)ws;
    ws += align256((size_t)a->bs * NR * sp.splits * sizeof(Partial));
    P.dec = (Dec*)ws;
    ws += align256((size_t)a->bs * sizeof(Dec));
    P.sums = (double*)ws;
    P.NR = NR; P.splits = sp.splits; P.chunk = sp.chunk;

    RowSet tr{a->logits, a->row_stride, a->row_base, a->n_logit_rows, a->n_slots, 0, a->ld, 1, nullptr, a->ld, 0};
    const bool at = aligned16(a->logits, a->row_stride, a->dtype);
    if (a->prof_begin) hipEventRecord((hipEvent_t)a->prof_begin, st);
    if (P.greedy) launch_stats<true>(a->dtype, at, tr, a->vocab, sp, a->bs, P.c, P.part, NR, st);
    else launch_stats<false>(a->dtype, at, tr, a->vocab, sp, a->bs, P.c, P.part, NR, st);
    if (!P.greedy && P.dlogits) {
        RowSet dr{a->draft_logits, a->draft_row_stride, a->draft_row_base, a->n_draft_rows, a->n_slots, 0, a->ld, 0,
                  a->slot_flags ? a->slot_flags : nullptr, a->ld, a->ld + 1};
        if (a->slot_flags) {
            const bool ad = aligned16(a->draft_logits, a->draft_row_stride, a->draft_dtype);
            launch_stats<false>(a->draft_dtype, ad, dr, a->vocab, sp, a->bs, P.c, P.part, NR, st);
        }
    }
    if (a->prof_end) hipEventRecord((hipEvent_t)a->prof_end, st);
    hipLaunchKernelGGL(k_decide, dim3(a->bs), dim3(kDecideBlock), 0, st, P);
    const bool need_final = !P.greedy || P.ctx;
    if (!P.greedy) {
        dim3 grid(sp.splits, a->bs);
        const int tt = a->dtype, dd = P.dlogits ? a->draft_dtype : a->dtype;
        if (tt == SPEC_F32 && dd == SPEC_F32) hipLaunchKernelGGL((k_sample_partial<SPEC_F32, SPEC_F32>), grid, dim3(kBlock), 0, st, P);
        else if (tt == SPEC_F32) hipLaunchKernelGGL((k_sample_partial<SPEC_F32, SPEC_BF16>), grid, dim3(kBlock), 0, st, P);
        else if (dd == SPEC_F32) hipLaunchKernelGGL((k_sample_partial<SPEC_BF16, SPEC_F32>), grid, dim3(kBlock), 0, st, P);
        else hipLaunchKernelGGL((k_sample_partial<SPEC_BF16, SPEC_BF16>), grid, dim3(kBlock), 0, st, P);
    }
    if (need_final) {
        const int tt = a->dtype, dd = P.dlogits ? a->draft_dtype : a->dtype;
        if (tt == SPEC_F32 && dd == SPEC_F32) hipLaunchKernelGGL((k_sample_final<SPEC_F32, SPEC_F32>), dim3(a->bs), dim3(kBlock), 0, st, P);
        else if (tt == SPEC_F32) hipLaunchKernelGGL((k_sample_final<SPEC_F32, SPEC_BF16>), dim3(a->bs), dim3(kBlock), 0, st, P);
        else if (dd == SPEC_F32) hipLaunchKernelGGL((k_sample_final<SPEC_BF16, SPEC_F32>), dim3(a->bs), dim3(kBlock), 0, st, P);
        else hipLaunchKernelGGL((k_sample_final<SPEC_BF16, SPEC_BF16>), dim3(a->bs), dim3(kBlock), 0, st, P);
    }
    return spec_record_hip_error(hipGetLastError());
}

int spec_verify_tree_launch(const spec_tree_verify_args* a, hipStream_t st)
{
    RowSplit sp = row_split(a->bs, a->vocab);
    TreeParams P;
    P.bs = a->bs; P.vocab = a->vocab; P.rows_max = a->rows_max;
    P.row_base = a->row_base; P.n_rows_buf = a->n_logit_rows;
    P.node_token = a->node_token; P.parent_row = a->parent_row; P.n_rows = a->n_rows;
    P.out_tokens = a->out_tokens; P.out_num = a->out_num; P.out_path = a->out_path_rows; P.out_argmax = a->out_argmax;
    P.out_flags = a->out_flags;
    P.ctx = a->ctx; P.ctx_stride = a->ctx_stride; P.ctx_len = a->ctx_len; P.ctx_cap = a->ctx_cap;
    P.part = (Partial*)a->workspace;
    P.splits = sp.splits;
    RowSet rs{a->logits, a->row_stride, a->row_base, a->n_logit_rows, a->n_rows, 1, a->rows_max, 0, nullptr, 0, 0};
    if (a->prof_begin) hipEventRecord((hipEvent_t)a->prof_begin, st);
    launch_stats<true>(a->dtype, aligned16(a->logits, a->row_stride, a->dtype), rs, a->vocab, sp, a->bs, 1.0f, P.part,
                       a->rows_max, st);
    if (a->prof_end) hipEventRecord((hipEvent_t)a->prof_end, st);
    hipLaunchKernelGGL(k_tree_walk, dim3(a->bs), dim3(kWave), 0, st, P);
    return spec_record_hip_error(hipGetLastError());
}
