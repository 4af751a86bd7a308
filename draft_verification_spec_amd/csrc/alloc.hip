// Verification-budget allocation.
//
// Chains (Hybrid Spark, Algorithm 1 and Sections 4.2-4.4), two launches:
//   k_alloc_slots: one wave per request evaluates every n-gram estimate
//     (Eq. (1)) and model confidence in fp64 on its lanes, forms the survival
//     running products, the chain values of Eq. (3) and the choice (contains
//     rule, value rule with ties to the n-gram chain, or a lossless policy of
//     Appendix H), and writes the chosen chain and one 64-bit ranking key per
//     slot: fp32(S) bits | (31 - position) | (2^27 - 1 - request), so the
//     largest key is "highest survival, then lower position, then lower
//     request" and keys are unique;
//   k_alloc_topk: one workgroup finds the exact budget-th largest key by an
//     8-bit radix select over an LDS histogram (the digit is found by a
//     wave-wide suffix scan), stopping as soon as the boundary bucket is taken
//     whole, then each request's verified prefix and the CSR row bases.
// Trees (AdaSpark, Sections 2.2, 3.1, 3.3):
//   k_tree    : four waves per request build the candidate forest (drafter
//               block + n-gram chains, copied or follower tokens) in one
//               parallel pass over the chains' tokens (or chain by chain on
//               wave 0 for the largest forests), then the acceptance
//               estimates of the Eq. (6) form, the path products Q, the
//               best-first top rows_cap-1 (Proposition 1) and the
//               depth-first layout.
//   k_tree_forest: the same rows from a forest the caller built.
//   k_rows_scan: exclusive prefix sum of the rows per request.
#include <cstring>

#include "common.hpp"

namespace spec {

constexpr int kAllocBlock = 1024;
constexpr int kSlotBlock = 256;                 // four requests (one wave each) per workgroup
constexpr int kSlotReqs = kSlotBlock / kWave;
constexpr int kLdsKeys = 4096;                  // ranking keys the select kernel keeps in LDS (32 KB)

struct SelectParams {
    spec_chain_alloc a;
    uint64_t* keys;  // [bs, ld] ranking keys, in the workspace
};

__device__ __forceinline__ double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

// A wave-uniform float as a scalar value: selecting between such values
// stays a select, where a select between two struct fields would become a
// per-lane load from the selected address.
__device__ __forceinline__ float sval(float x)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Eq. (1) logit of position k (1-based); `lnm` = ln(min(max(m,1), m_cap) / m_ref).
__device__ __forceinline__ double est_logit(const spec_estimator& e, int k, int n, int a, double lnm)
{
    const bool first = (k == 1);
    const int bi = (k <= 15 ? k : 15) - 1;
    float beta = sval(e.beta[0]);
#pragma unroll
    for (int i = 1; i < 15; ++i) beta = bi == i ? sval(e.beta[i]) : beta;
    double z = (double)beta + (double)(first ? sval(e.w_first) : sval(e.w_rest)) * ((double)n - (double)e.n_ref) +
               (double)e.delta * (double)a;
    if ((double)n >= (double)e.n_full)
        z += (double)(first ? sval(e.l_first) : sval(e.l_rest)) + (double)(first ? sval(e.k_first) : sval(e.k_rest)) * lnm;
    return z;
}

// Lane k's double, broadcast to the wave (k wave-uniform).
__device__ __forceinline__ double lane_value(double v, int k)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), k);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), k);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// One wave per request.  Lane k evaluates slot k's n-gram estimate (Eq. (1))
// and model confidence in fp64; the survival running products, the chain
// values of Eq. (3) and the choice (contains rule, value rule with ties to the
// n-gram chain, or a lossless policy of Appendix H) are then computed by every
// lane alike, as the same left folds the definition uses, with lane k's values
// broadcast in turn; finally lane k writes slot k of the chosen chain and its
// ranking key.
__global__ __launch_bounds__(kSlotBlock) void k_alloc_slots(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int lane = threadIdx.x % kWave;
    const int r = blockIdx.x * kSlotReqs + (int)(threadIdx.x / kWave);
    if (r >= A.bs) return;   // the whole wave (no workgroup barrier in this kernel)
    const int K = A.K, ld = A.ld;
    const int gcap = A.ngram_ld < ld ? A.ngram_ld : ld;
    const int k = lane;
    // Every input first, from in-bounds addresses, and all of them in one
    // round trip: otherwise the compiler sinks each load into the branch that
    // uses it, one dependent trip after another.
    const int kc = k < K ? k : (K > 0 ? K - 1 : 0);
    const int gc = k < gcap ? k : (gcap > 0 ? gcap - 1 : 0);
    const int rl0 = A.ngram_len[r];
    const int n0 = A.ngram_feat[4 * (int64_t)r + 0];
    const int am0 = A.ngram_feat[4 * (int64_t)r + 1];
    const int mf0 = A.ngram_feat[4 * (int64_t)r + 2];
    const int32_t td0 = K > 0 ? A.model_tokens[(int64_t)r * K + kc] : -1;
    const float cv0 = K > 0 ? A.model_conf[(int64_t)r * K + kc] : 0.0f;
    const int32_t tg0 = gcap > 0 ? A.ngram_draft[(int64_t)r * A.ngram_ld + gc] : -1;
    const int pm1 = A.model_point_mass ? (int)A.model_point_mass[r] : 1;
    asm volatile("" : : "v"(rl0), "v"(n0), "v"(am0), "v"(mf0), "v"(td0), "v"(cv0), "v"(tg0), "v"(pm1));
    // the request's own words are the same on every lane: as scalars, the
    // chain lengths make the folds below uniform loops and branches
    const int rl = __builtin_amdgcn_readfirstlane(rl0), n = __builtin_amdgcn_readfirstlane(n0);
    const int am = __builtin_amdgcn_readfirstlane(am0), mf = __builtin_amdgcn_readfirstlane(mf0);
    const int pm0 = __builtin_amdgcn_readfirstlane(pm1);
    const int glen = rl < 0 ? 0 : (rl > gcap ? gcap : rl);
    double mm = (double)mf;
    mm = mm < 1.0 ? 1.0 : (mm > (double)A.est.m_cap ? (double)A.est.m_cap : mm);
    const double lnm = ((double)n >= (double)A.est.n_full) ? log(mm / (double)A.est.m_ref) : 0.0;
    const bool mpm = pm0 != 0;
    int32_t td = -1, tg = -1;
    double h = 0.0, c = 0.0;
    if (k < K) {
        td = td0;
        const double cv = (double)cv0;
        c = A.conf_is_logit ? sigm(cv) : cv;
    }
    if (k < gcap) tg = tg0;
    if (k < glen) h = sigm(est_logit(A.est, k + 1, n, am, lnm));
    const bool mismatch = __ballot(k < K && td != tg) != 0;
    // chain values (Eq. (3)) from the running products, both chains in one
    // loop (independent folds); lane q keeps the products after term q, and
    // every lane the ones after term K-1
    const double lam = (double)A.lambda;
    double sg = 1.0, sd = 1.0, vg = 0.0, vd = 0.0;
    double mg = 0.0, md = 0.0, sgK = 1.0, sdK = 1.0;
    const int qn = glen > K ? glen : K;
    for (int q = 0; q < qn; ++q) {
        if (q < glen) {
            sg *= lane_value(h, q);
            vg += sg > lam ? sg - lam : 0.0;
        }
        if (q < K) {
            sd *= lane_value(c, q);
            vd += sd > lam ? sd - lam : 0.0;
        }
        if (lane == q) { mg = sg; md = sd; }
        if (q == K - 1) { sgK = sg; sdK = sd; }
    }
    const bool prefix = glen > K && !mismatch;
    int use = SPEC_SRC_MODEL;
    switch (A.policy) {
    case SPEC_POLICY_PROPOSED:
        if (prefix) use = SPEC_SRC_MERGED;
        else if (glen >= 1) use = vg >= vd ? SPEC_SRC_NGRAM : SPEC_SRC_MODEL;
        break;
    case SPEC_POLICY_NGRAM_FIRST: use = glen >= 1 ? SPEC_SRC_NGRAM : SPEC_SRC_MODEL; break;
    case SPEC_POLICY_EXTENSION: use = prefix ? SPEC_SRC_EXTENDED : SPEC_SRC_MODEL; break;
    case SPEC_POLICY_NGRAM_ONLY: use = SPEC_SRC_NGRAM; break;
    default: use = SPEC_SRC_MODEL;
    }
    const int len = (use == SPEC_SRC_MODEL) ? K : glen;
    // Survival S_k of the chosen chain on lane k: the model or n-gram running
    // product, the larger of the two on the shared prefix of a merged chain
    // (the model's on an extended one), and past slot K-1 of those the prefix
    // value times h_K ... h_k, multiplied in that order.
    double mine;
    if (use == SPEC_SRC_MODEL) mine = md;
    else if (use == SPEC_SRC_NGRAM) mine = mg;
    else {
        const bool ext = use == SPEC_SRC_EXTENDED;
        mine = (lane < K) ? (ext ? md : (mg > md ? mg : md)) : (K > 0 ? (ext ? sdK : (sgK > sdK ? sgK : sdK)) : 1.0);
        for (int q = K; q < len; ++q) {
            const double hq = lane_value(h, q);
            if (q <= lane) mine *= hq;
        }
    }
    if (lane >= len) mine = 0.0;
    if (k < ld) {
        int32_t tk = -1;
        uint8_t fl = 0;
        if (k < len) {
            const bool model_slot = use == SPEC_SRC_MODEL || (use == SPEC_SRC_EXTENDED && k < K);
            tk = (use == SPEC_SRC_MODEL) ? td : tg;
            fl = model_slot ? (mpm ? SPEC_SLOT_POINT_MASS : 0) : (SPEC_SLOT_POINT_MASS | SPEC_SLOT_FROM_NGRAM);
        }
        const int64_t o = (int64_t)r * ld + k;
        A.chain_tokens[o] = tk;
        A.slot_flags[o] = fl;
        A.survival[o] = (float)mine;
        // fp32(S) bits | (31 - position) | (2^27 - 1 - request): the largest key
        // is "highest survival, then lower position, then lower request"
        P.keys[o] = (k < len) ? (((uint64_t)__float_as_uint((float)mine) << 32) | ((uint64_t)(31 - k) << 27) |
                                 (uint64_t)(0x7FFFFFF - r))
                              : 0ull;
    }
    if (lane == 0) {
        A.chain_len[r] = len;
        A.chain_src[r] = use;
        A.out_flags[r] = (rl < 0 || rl > gcap) ? SPEC_FLAG_BAD_LENGTH : 0u;
    }
}

// Exclusive prefix over a workgroup of kAllocBlock threads (the size is a
// constant: blockDim is a load from the dispatch packet).
__device__ int64_t block_exclusive_i64(int64_t v, int64_t* total)
{
    __shared__ int64_t sh[32];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    constexpr int nw = kAllocBlock / kWave;
    int64_t inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int64_t u = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += u;
    }
    __syncthreads();
    if (lane == kWave - 1) sh[wid] = inc;
    __syncthreads();
    int64_t before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        if (w < wid) before += sh[w];
        tot += sh[w];
    }
    *total = tot;
    return before + inc - v;
}

// Exclusive prefix over a workgroup of kAllocBlock threads of 32-bit
// counts; *total gets the sum.
__device__ uint32_t block_exclusive_u32(uint32_t v, uint32_t* total)
{
    __shared__ uint32_t sh[32];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    constexpr int nw = kAllocBlock / kWave;
    const uint32_t inc = wave_incl_add(v);
    __syncthreads();
    if (lane == kWave - 1) sh[wid] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        if (w < wid) before += sh[w];
        tot += sh[w];
    }
    *total = tot;
    return before + inc - v;
}

// Histogram increment with the lanes that share the first active lane's digit
// folded into one LDS atomic (at the top digits nearly every key agrees).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, int dg)
{
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const int ldg = __builtin_amdgcn_readlane(dg, leader);
    const uint64_t peers = __ballot(active && dg == ldg);
    const int lane = threadIdx.x % kWave;
    if (lane == leader) atomicAdd(&hist[ldg], (uint32_t)__popcll(peers));
    else if (active && dg != ldg) atomicAdd(&hist[dg], 1u);
}

// The threshold of the budget largest ranking keys by an 8-bit radix select over the
// survival and position bytes (stopping as soon as the boundary bucket is
// taken whole), the request bits by one ordered scan, then each request's
// verified prefix and the row bases.  One workgroup.
__global__ __launch_bounds__(kAllocBlock) void k_alloc_topk(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int bs = A.bs, ld = A.ld;
    const int64_t N = (int64_t)bs * ld;
    __shared__ uint64_t lkeys[kLdsKeys];
    // one histogram per wave (double-buffered): at the top digits nearly every
    // key agrees, and atomics of all waves on one LDS word serialize
    __shared__ __align__(16) uint32_t hist[2][kAllocBlock / kWave][256];
    __shared__ uint64_t sh_prefix;
    __shared__ int64_t sh_rem, sh_valid;
    __shared__ int sh_done;
    const bool in_lds = N <= kLdsKeys;
    const int wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) { sh_prefix = 0; sh_valid = 0; sh_done = 0; }
    {
        int64_t valid = 0;
        for (int64_t i = threadIdx.x; i < N; i += kAllocBlock) {
            const uint64_t k = P.keys[i];
            if (in_lds) lkeys[i] = k;
            valid += k != 0;
        }
        valid = wave_sum(valid);
        __syncthreads();   // sh_valid initialised
        if (lane == 0) atomicAdd((unsigned long long*)&sh_valid, (unsigned long long)valid);
    }
    __syncthreads();
    // The selection, instantiated once for keys in LDS and once for keys in
    // global memory, so that each reads through its own address space (a
    // pointer that may be either compiles to flat loads, which wait for every
    // outstanding access).
    auto select = [&](const uint64_t* keys) __attribute__((always_inline)) {
    const int64_t take = (A.budget < sh_valid) ? A.budget : sh_valid;
    uint64_t theta = ~0ull;  // nothing selected
    if (take > 0) {
        if (threadIdx.x == 0) sh_rem = take;
        uint64_t mask = 0;
        for (int i = lane; i < 256; i += kWave) hist[0][wid][i] = 0;
        __syncthreads();
        for (int shift = 56, hb = 0; shift >= 0; shift -= 8, hb ^= 1) {
            // the histogram of this pass was cleared during the previous one
            uint32_t* H = hist[hb][wid];
            const uint64_t pre = sh_prefix;
            const int64_t rounds = (N + kAllocBlock - 1) / kAllocBlock;
            for (int64_t u = 0; u < rounds; ++u) {
                const int64_t i = threadIdx.x + u * kAllocBlock;
                const uint64_t k = i < N ? keys[i] : 0ull;
                hist_add(H, k != 0 && (k & mask) == pre, (int)((k >> shift) & 255u));
            }
            for (int i = lane; i < 256; i += kWave) hist[hb ^ 1][wid][i] = 0;
            __syncthreads();
            if (wid == 0) {
                // lane l owns digits 255-4l .. 252-4l (descending); suffix counts from the top
                // (each digit's count summed over the waves' histograms)
                uint32_t c4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int w = 0; w < kAllocBlock / kWave; ++w) {
                    const uint4 q = *(const uint4*)&hist[hb][w][252 - 4 * lane];
                    c4[0] += q.w; c4[1] += q.z; c4[2] += q.y; c4[3] += q.x;
                }
                const uint32_t own = c4[0] + c4[1] + c4[2] + c4[3];
                const uint32_t inc = wave_incl_add(own);
                const int64_t rem = sh_rem;
                const int64_t above = (int64_t)(inc - own);
                if (above < rem && (int64_t)inc >= rem) {
                    int64_t cum = above;
                    for (int j = 0; j < 4; ++j) {
                        if (cum + c4[j] >= rem) {
                            sh_rem = rem - cum;
                            sh_prefix = pre | ((uint64_t)(255 - 4 * lane - j) << shift);
                            // every key of the boundary bucket is taken: the threshold is its smallest key
                            sh_done = (cum + c4[j] == rem);
                            break;
                        }
                        cum += c4[j];
                    }
                }
            }
            mask |= 255ull << shift;
            __syncthreads();
            if (sh_done) break;
            if (shift == 24) {
                // Survival and position are fixed: at most one key per
                // request matches the prefix, and index order is request
                // order, i.e. descending key order.  The threshold is the
                // rem-th match in index order: one scan instead of three
                // more passes.
                const uint64_t pre2 = sh_prefix;
                const int64_t per = (N + kAllocBlock - 1) / kAllocBlock;
                const int64_t i0 = (int64_t)threadIdx.x * per;
                uint32_t cnt = 0;
                for (int64_t i = i0; i < i0 + per && i < N; ++i) {
                    const uint64_t k = keys[i];
                    cnt += (k != 0 && (k & mask) == pre2);
                }
                uint32_t all;
                int64_t before = block_exclusive_u32(cnt, &all);
                const int64_t rem = sh_rem;
                if (before < rem && before + cnt >= rem) {
                    for (int64_t i = i0; i < i0 + per && i < N; ++i) {
                        const uint64_t k = keys[i];
                        if (k != 0 && (k & mask) == pre2 && ++before == rem) sh_prefix = k;
                    }
                }
                mask = ~0ull;
                __syncthreads();
                break;
            }
        }
        // the threshold: the boundary key, or, when the boundary bucket is
        // taken whole, its prefix with the lower bits zero (every key of the
        // bucket is at least that, every key below the bucket less)
        theta = sh_prefix;
    }
    // verified prefix per request, row bases over (alloc + 1).  A request's
    // keys are read in batches of 16 from clamped (in-bounds) positions, so
    // that each batch is one round of loads; a thread with several requests
    // counts them again for the row bases rather than rereading alloc_len.
    const int per = (bs + kAllocBlock - 1) / kAllocBlock;
    const int r0 = threadIdx.x * per;
    auto count_of = [&](int r) -> int {
        int cnt = 0;
        for (int k0 = 0; k0 < ld; k0 += 16) {
            uint64_t kv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) kv[j] = keys[(int64_t)r * ld + (k0 + j < ld ? k0 + j : k0)];
#pragma unroll
            for (int j = 0; j < 16; ++j) cnt += (k0 + j < ld && kv[j] != 0 && kv[j] >= theta);
        }
        return cnt;
    };
    uint32_t local = 0;
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        const int cnt = count_of(r);
        A.alloc_len[r] = cnt;
        local += cnt + 1;
    }
    uint32_t total;
    int64_t base = block_exclusive_u32(local, &total);
    if (per == 1) {
        if (r0 < bs) A.row_base[r0] = base;
    } else {
        for (int r = r0; r < r0 + per && r < bs; ++r) {
            A.row_base[r] = base;
            base += count_of(r) + 1;
        }
    }
    if (threadIdx.x == 0) A.total_rows[0] = (int32_t)total;
    };
    if (in_lds) select(lkeys);
    else select(P.keys);
}

// ---------------------------------------------------------------------------
// trees
// ---------------------------------------------------------------------------

struct TreeBuildParams {
    spec_tree_alloc a;
    spec_tree_scores sc;   // copied from a.scores when given
    int32_t scored;
};

__device__ __forceinline__ double clamp_prob(double x) { return x < 1e-6 ? 1e-6 : (x > 1.0 - 1e-6 ? 1.0 - 1e-6 : x); }
__device__ __forceinline__ double logit_prob(double x) { x = clamp_prob(x); return log(x / (1.0 - x)); }

// Evidence class of a follower count l >= 1: floor(log2 l), at most 7.
__device__ __forceinline__ int follower_class(int l) { return l <= 1 ? 0 : min(7, 31 - __clz(l)); }

// Evidence class of an n-gram chain: floor(log2) of its source's match
// length (feature m, else n), at most 7.
__device__ __forceinline__ int evidence_of(const int32_t* feat)
{
    const int l = feat[2] > 0 ? feat[2] : feat[0];
    return l <= 1 ? 0 : min(7, 31 - __clz(l));
}

// A double from lane l (wave-uniform l), and a double from lane l of each lane's choosing.
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double shfl_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)b, l, kWave);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(b >> 32), l, kWave);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// A global-memory int32 pointer, kept apart from LDS pointers.
typedef const __attribute__((address_space(1))) int32_t* gi32_ptr;

// Best-first rank of nodes 1..cnt-1 by (fp32 Q descending, index ascending),
// S(n), the depth-first layout of the chosen set and the request's outputs
// ([AS] Section 3.1).  The forest's tokens, parents and Q are in LDS, with
// fsel zero for every node; every thread of the workgroup (one request)
// calls it: the ranks are shared out over all of them, the layout is wave
// 0's, S(n) wave 1's (wave 0's in a one-wave workgroup), and flags are
// thread 0's.
__device__ __forceinline__ void tree_rows(const spec_tree_alloc& A, int r, int lane, int cnt, uint32_t flags,
                                          const int32_t* ftok, const int32_t* fpar, const double* fQ, uint8_t* fsel)
{
    __shared__ double sQrank[SPEC_MAX_ROWS];
    const int t = threadIdx.x, nthr = blockDim.x;
    const bool w0 = t < kWave;
    // best-first: rank by (fp32 Q desc, index asc); keep rank < rows_cap - 1
    const int keep = A.rows_cap - 1;
    if (cnt <= kWave) {
        // a forest within one wave: the keys in registers, node j on lane j
        if (w0) {
            const bool mine = lane >= 1 && lane < cnt;
            const double qj = mine ? fQ[lane] : 0.0;
            const uint64_t kj = mine ? ((uint64_t)__float_as_uint((float)qj) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)lane) : 0;
            // (lanes outside 1..cnt-1 hold key 0, which outranks nothing: the
            // loop runs over every lane with constant lane indices)
            int rank = 0;
#pragma unroll
            for (int i = 1; i < kWave; ++i) {
                const uint64_t ki = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(kj >> 32), i) << 32)
                                  | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kj, i);
                rank += ki > kj;
            }
            if (mine) {
                fsel[lane] = rank < keep;
                if (rank < A.rows_cap) sQrank[rank] = qj;
            }
        }
    } else for (int j = 1 + t; j < cnt; j += nthr) {
        const uint64_t kj = ((uint64_t)__float_as_uint((float)fQ[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        int rank = 0;
        for (int i = 1; i < cnt; ++i) {
            const uint64_t ki = ((uint64_t)__float_as_uint((float)fQ[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
            rank += ki > kj;
        }
        fsel[j] = rank < keep;
        if (rank < A.rows_cap) sQrank[rank] = fQ[j];
    }
    // Depth-first layout, children in index order.  The selected nodes (the
    // anchor and at most rows_cap - 1 candidates) are compacted in index
    // order, node i on lane i; a parent precedes its children in that order.
    // Each lane's row is then the number of nodes that precede it depth-first:
    // its ancestors, and every node whose path leaves their deepest common
    // ancestor through a lower-index child.
    __shared__ int32_t scomp[SPEC_MAX_ROWS];      // compact position -> forest node
    __shared__ int32_t scpar[SPEC_MAX_ROWS];      // compact position -> its node's parent
    __shared__ int16_t scpos[SPEC_MAX_FOREST];    // forest node -> compact position
    if (t == 0) fsel[0] = 1;
    __syncthreads();
    int m = 0;
    for (int base = 0; w0 && base < cnt; base += kWave) {
        const int c = base + lane;
        const bool sel = c < cnt && fsel[c];
        const uint64_t bal = __ballot(sel);
        const int at = m + (int)__popcll(bal & ((1ull << lane) - 1ull));
        if (sel && at < SPEC_MAX_ROWS) {
            scomp[at] = c;
            scpar[at] = c > 0 ? fpar[c] : -1;
            scpos[c] = (int16_t)at;
        }
        m += (int)__popcll(bal);
    }
    // m as a scalar: the loop above runs on wave 0 only, which the compiler
    // cannot tell, and the layout walk below would otherwise run divergent
    m = __builtin_amdgcn_readfirstlane(m < A.rows_cap ? m : A.rows_cap);
    __syncthreads();
    if (A.s_curve && (nthr > kWave ? (t >= kWave && t < 2 * kWave) : w0)) {
        // S(n): the first n - 1 nodes of the best-first order, accumulated in
        // order (lane n - 1 holds the (n - 1)-th Q); on the second wave when
        // there is one, beside wave 0's layout
        const double v = (lane < A.rows_cap && lane < cnt - 1) ? sQrank[lane] : 0.0;
        double acc = 0.0, mine = 0.0;
        for (int n = 1; n <= A.rows_cap; ++n) {
            mine = lane == n - 1 ? acc : mine;
            if (n - 1 < cnt - 1) acc += readlane_f64(v, n - 1);
        }
        if (lane < A.rows_cap) A.s_curve[(int64_t)r * A.rows_cap + lane] = (float)mine;
    }
    if (!w0) return;
    const bool in = lane < m;
    const int mynode = in ? scomp[lane] : -1;
    // the parent's compact position (-1 at the anchor; -2 for a parent left
    // out of the set, which cuts the node and its subtree off the layout;
    // -3 past the set)
    int jmp = in ? -1 : -3;
    if (in && lane > 0) {
        const int pf = scpar[lane];
        jmp = fsel[pf] ? (int)scpos[pf] : -2;
    }
    const int up = jmp;
    // ancestors-or-self as a lane mask, by pointer doubling: anc holds the
    // first nodes of the path up from the lane and jmp the next one above
    // them (-1: the anchor was reached)
    uint64_t anc = in ? (1ull << lane) : 0ull;
    while (__builtin_amdgcn_ballot_w64(jmp >= 0)) {
        const int src = jmp >= 0 ? jmp : lane;
        const uint64_t a2 = ((uint64_t)(uint32_t)__shfl((int)(anc >> 32), src, kWave) << 32)
                          | (uint32_t)__shfl((int)(uint32_t)anc, src, kWave);
        const int j2 = __shfl(jmp, src, kWave);
        if (jmp >= 0) {
            anc |= a2;
            jmp = j2;
        }
    }
    const bool reach = in && jmp == -1;
    // The nodes before this one: w is an ancestor (w's set within ours), or
    // both paths continue below the common ancestor and w's continues through
    // the lower index (along a path the indices grow with depth, so the
    // lowest index of a path's part below the common ancestor is its child
    // there).  With lowest(empty) = -1 one signed compare decides: an
    // ancestor has x empty (-1 < anything), a descendant has y empty (never
    // before).  Four lanes w per round (lanes past the set hold jmp -3 and
    // never count).
    int row = 0;
    for (int wb = 0; wb < m; wb += 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int w = wb + k;
            const uint64_t aw = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(anc >> 32), w) << 32)
                              | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)anc, w);
            const int jw = __builtin_amdgcn_readlane(jmp, w);
            const int cx = __ffsll((unsigned long long)(aw & ~anc)) - 1;
            const int cy = __ffsll((unsigned long long)(anc & ~aw)) - 1;
            row += (int)((jw == -1) & (w != lane) & (cx < cy));
        }
    }
    const int prow = __shfl(row, up < 0 ? 0 : up, kWave);
    const int nrows = (int)__popcll(__builtin_amdgcn_ballot_w64(reach));
    int32_t* nt = A.node_token + (int64_t)r * A.rows_cap;
    int32_t* pr = A.parent_row + (int64_t)r * A.rows_cap;
    float* Qo = A.Q + (int64_t)r * A.rows_cap;
    if (reach) {
        nt[row] = (mynode == 0) ? -1 : ftok[mynode];
        pr[row] = lane == 0 ? -1 : prow;
        Qo[row] = (float)fQ[mynode];
    }
    if (lane >= nrows && lane < A.rows_cap) {
        nt[lane] = -1; pr[lane] = -1; Qo[lane] = 0.0f;
    }
    if (t == 0) {
        A.n_rows[r] = nrows;
        A.forest_count[r] = cnt;
        A.out_flags[r] = flags;
    }
}

// An int32 view of LDS scratch that the walk borrows from arrays written only
// after it.
typedef int32_t __attribute__((may_alias)) wi32;

// The parallel walk's words, in LDS borrowed from an array written only after
// the walk: a drafter node's largest passing bucket (-1: none), and per chain
// its entries (tokens within the depth limit), first entry off the pick path,
// entries that are drafter nodes, depth of its first own node (kWalkNone:
// none), index of its first own node; then the own nodes of all chains.
constexpr int kWalkPass = 1 << 20;   // on a made node's entry: a later chain passes it
constexpr int kWalkNone = 1 << 30;
struct WalkWords {
    wi32 *pass, *geff, *fp, *ndr, *dn, *base, *total;
    __device__ explicit WalkWords(wi32* w)
        : pass(w), geff(w + SPEC_MAX_FOREST), fp(geff + kWave), ndr(fp + kWave), dn(ndr + kWave),
          base(dn + kWave), total(base + kWave) {}
};

// The parallel walk's starting values, set before the workgroup's first
// barrier (the chain lengths are read from memory: their LDS copy is being
// written meanwhile): the per-chain words on wave 0, the marks and the pairs'
// agreement lengths by every thread.
__device__ __forceinline__ void walk_parallel_init(const spec_tree_alloc& A, int P_, int nd, int64_t q0, int nthr,
                                                   wi32* wagr, wi32* wscr, uint32_t& flags)
{
    const WalkWords W(wscr);
    const int t = threadIdx.x, lane = t % kWave;
    const int L = A.ngram_ld, C = P_ + 1, npair = C * (C - 1) / 2;
    if (t < kWave) {
        const int gl = lane < C ? A.ngram_len[q0 + lane] : 0;
        if (__builtin_amdgcn_ballot_w64(gl < 0 || gl > L)) flags |= SPEC_FLAG_BAD_LENGTH;
        if (lane < C) {
            const int g = gl < 0 ? 0 : (gl > L ? L : gl);
            int ge = A.depth_max - lane < g ? A.depth_max - lane : g;
            ge = ge > 0 ? ge : 0;
            W.geff[lane] = ge;
            W.fp[lane] = ge;
            W.ndr[lane] = ge;
            W.dn[lane] = kWalkNone;
        }
    }
    for (int n = t; n < nd; n += nthr) W.pass[n] = -1;
    for (int q = t; q < npair; q += nthr) wagr[q] = kWalkNone;
}

// The chain walk without a walk: every (chain, token) entry finds its node at
// once, over the whole workgroup.  Chain c starts at the anchor (c = 0, depth
// 0) or at pick c (depth c); its token i sits at depth c + 1 + i.  A node is
// fixed by the tokens on its path from the anchor, so:
//   - entries before fp_c, the chain's first token off the pick path, are the
//     picks of their positions (the lowest candidate holding a pick's token is
//     the pick itself); the entry at fp_c, if its position is in the block, is
//     the lowest other candidate holding its token, if any; every later entry
//     is an n-gram node (neither a sibling nor an n-gram node has drafter
//     children);
//   - two chains c' < c reach the same n-gram node at depth d exactly when c'
//     passes pick c and their tokens agree from depth c + 1 to d: the node was
//     made by the lowest such c' (c itself if none).
// A chain's own nodes are the tail of its entries; they are numbered in chain
// order and then depth order, the order a chain-by-chain walk appends them in,
// so c_max keeps the same ones.  A node passed by a later chain is marked
// agreed; a drafter node also takes the largest bucket of the tokens that pass
// it.  All threads of the workgroup call this (it holds barriers); the drafter
// nodes are in the forest arrays already.  Writes the n-gram nodes and the
// marks and returns the node count.  Its starting values come from
// walk_parallel_init, before the barrier this begins after.
__device__ __forceinline__ int walk_parallel(const spec_tree_alloc& A, int P_, int Kc, int nd, int cmax, int nthr,
                                             const int8_t* cev, const int32_t* ctok,
                                             const int32_t* cfol, int32_t* ftok, int32_t* fpar, int32_t* fdep,
                                             uint8_t* fkind, int8_t* fabove, int8_t* fbucket, int8_t* fagree,
                                             wi32* went, wi32* wagr, wi32* wscr)
{
    constexpr int kPass = kWalkPass, kNone = kWalkNone;
    const WalkWords W(wscr);
    wi32* wpass = W.pass;
    wi32* cgeff = W.geff;
    wi32* cfp = W.fp;
    wi32* cndr = W.ndr;
    wi32* cdn = W.dn;
    wi32* cbase = W.base;
    wi32* ctotal = W.total;
    const int t = threadIdx.x, lane = t % kWave;
    const int L = A.ngram_ld, C = P_ + 1, E = C * L, npair = C * (C - 1) / 2;
    const bool w0 = t < kWave;
    // x / L for 0 <= x < 2^20 as a multiply-high by ceil(2^32 / L) (exact:
    // the error is below x / 2^32, less than the distance to the next
    // multiple of 1 / L); L = 1 apart, whose factor does not fit 32 bits
    const uint32_t mL = L > 1 ? 0xFFFFFFFFu / (uint32_t)L + 1u : 0u;
    auto divL = [&](int x) { return L > 1 ? (int)__umulhi((uint32_t)x, mL) : x; };
    const int pick0 = 1;   // node of position d's pick: pick0 + (d - 1) * Kc
    // departures from the pick path, and the pairs' agreement lengths (pair
    // (c', c), c' < c, at c (c - 1) / 2 + c': the first j at which chain c's
    // token j and chain c''s token at the same depth differ or either ends)
    for (int e = t; e < E; e += nthr) {
        const int c = divL(e), i = e - c * L;
        if (i >= cgeff[c]) continue;
        const int d = c + 1 + i;
        if (d > P_ || ctok[e] != ftok[pick0 + (d - 1) * Kc]) atomicMin(&cfp[c], i);
    }
    for (int w = t; w < npair * L; w += nthr) {
        const int q = divL(w), j = w - q * L;
        // c with c (c - 1) / 2 <= q < (c + 1) c / 2
        int c = (int)((1.0f + sqrtf(1.0f + 8.0f * (float)q)) * 0.5f);
        c = c * (c - 1) / 2 > q ? c - 1 : ((c + 1) * c / 2 <= q ? c + 1 : c);
        const int cp = q - c * (c - 1) / 2, jp = c - cp + j;
        const bool differ = j >= cgeff[c] || jp >= cgeff[cp] || ctok[c * L + j] != ctok[cp * L + jp];
        if (differ) atomicMin(&wagr[q], j);
    }
    __syncthreads();
    // each entry's node: a drafter node's index, or 1024 + the chain that
    // makes the n-gram node
    for (int e = t; e < E; e += nthr) {
        const int c = divL(e), i = e - c * L;
        if (i >= cgeff[c]) continue;
        const int d = c + 1 + i, fp = cfp[c];
        int code = -1;
        if (i < fp) {
            code = pick0 + (d - 1) * Kc;
        } else if (i == fp && d <= P_) {
            const int tk = ctok[e];
            for (int k = 1; k < Kc; ++k)
                if (ftok[pick0 + (d - 1) * Kc + k] == tk) {
                    code = pick0 + (d - 1) * Kc + k;
                    break;
                }
        }
        if (i == fp) cndr[c] = fp + (code >= 0 ? 1 : 0);
        if (code >= 0) {
            const int fc = cfol[e];
            atomicMax(&wpass[code], fc > 0 ? 32 + 4 * follower_class(fc) : 4 * (int)cev[c]);
        } else {
            // (every earlier chain is looked at, with no early exit, so that
            // the loads go out together)
            int cr = c;
            for (int cp = c - 1; cp >= 0; --cp)
                if (cfp[cp] >= c - cp && wagr[c * (c - 1) / 2 + cp] >= d - c) cr = cp;
            code = 1024 + cr;
            if (cr == c) atomicMin(&cdn[c], d);
        }
        went[e] = code;
    }
    __syncthreads();
    // passes of other chains' nodes; the chains' first indices
    for (int e = t; e < E; e += nthr) {
        const int c = divL(e), i = e - c * L;
        if (i >= cgeff[c]) continue;
        const int code = went[e] & ~kPass;   // (another thread may be marking this entry)
        if (code >= 1024 && code - 1024 != c) {
            const int cr = code - 1024, d = c + 1 + i;
            atomicOr(&went[cr * L + (d - cr - 1)], kPass);
        }
    }
    if (w0) {
        const int dn = lane < C ? cdn[lane] : kNone;
        const int nnew = dn < kNone ? cgeff[lane] - (dn - lane - 1) : 0;
        int incl = nnew;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
        }
        if (lane < C) cbase[lane] = nd + incl - nnew;
        if (lane == kWave - 1) ctotal[0] = incl;
    }
    __syncthreads();
    // the new nodes
    for (int e = t; e < E; e += nthr) {
        const int c = divL(e), i = e - c * L;
        if (i >= cgeff[c]) continue;
        const int code = went[e];
        if ((code & ~kPass) != 1024 + c) continue;
        const int d = c + 1 + i, dn = cdn[c], idx = cbase[c] + (d - dn);
        if (idx >= cmax) continue;
        int par = idx - 1;
        if (i == 0) {
            par = c == 0 ? 0 : pick0 + (c - 1) * Kc;
        } else if (d == dn) {
            const int pc = went[e - 1] & ~kPass;
            par = pc < 1024 ? pc : cbase[pc - 1024] + (d - 1 - cdn[pc - 1024]);
        }
        const int ui = i - cndr[c];
        const int fc = cfol[e];
        ftok[idx] = ctok[e];
        fpar[idx] = par;
        fdep[idx] = d;
        fkind[idx] = (uint8_t)(3 | ((code & kPass) ? 4 : 0));
        fabove[idx] = (int8_t)(ui < 127 ? ui : 127);
        fbucket[idx] = (int8_t)((fc > 0 ? 32 + 4 * follower_class(fc) : 4 * (int)cev[c]) + (ui < 3 ? ui : 3));
        fagree[idx] = -1;
    }
    for (int n = t; n < nd; n += nthr) {
        const int b = wpass[n];
        if (b >= 0) {
            fkind[n] = (uint8_t)(fkind[n] | 4);
            fagree[n] = (int8_t)b;
        }
    }
    const int total = ctotal[0];
    return nd + total < cmax ? nd + total : cmax;
}

// Four waves per request.  The chain walk is walk_parallel's pass over the
// (chain, token) entries, or, for the largest forests and chains not staged
// in LDS, a chain-by-chain walk on wave 0 with forest node j in lane
// registers (lane j % 64, slot j / 64; NS * 64 >= c_max).  The weights,
// denominators and ranks of large forests are shared out over all four.
constexpr int kTreeBlock = 256;

template <int NS>
__global__ __launch_bounds__(kTreeBlock) void k_tree(TreeBuildParams P)
{
    const spec_tree_alloc& A = P.a;
    const int r = blockIdx.x, t = threadIdx.x, lane = t % kWave, wid = t / kWave;
    __shared__ int32_t ftok[SPEC_MAX_FOREST];
    __shared__ int32_t fpar[SPEC_MAX_FOREST];
    __shared__ int32_t fdep[SPEC_MAX_FOREST];
    __shared__ double fden[SPEC_MAX_FOREST];
    __shared__ double fQ[SPEC_MAX_FOREST];
    __shared__ uint8_t fsel[SPEC_MAX_FOREST];
    // Eq. (6) scoring state: kind (1 pick, 2 sibling, 3 n-gram; +4 agreed),
    // n-gram nodes above, an n-gram node's bucket, a drafter node's largest
    // agreeing bucket (-1 none), the weights exp(s)
    __shared__ uint8_t fkind[SPEC_MAX_FOREST];
    __shared__ int8_t fabove[SPEC_MAX_FOREST];
    __shared__ int8_t fbucket[SPEC_MAX_FOREST];
    __shared__ int8_t fagree[SPEC_MAX_FOREST];
    __shared__ int32_t fcontra[SPEC_MAX_FOREST];   // a drafter node's largest contradicting class (-1 none)
    __shared__ double fw[SPEC_MAX_FOREST];
    __shared__ unsigned long long fkids[kWave];   // a small forest's children, as lane masks
    // the Eq. (6) tables that nodes index by bucket, class or depth, copied
    // at the start (their per-lane reads would otherwise wait on memory after
    // the walk): buckets 64, agreements 64 x 2, contradictions 8 x 2, depths 16
    constexpr int kCoefAg = 64, kCoefCo = kCoefAg + 128, kCoefPsi = kCoefCo + 16, kCoefN = kCoefPsi + 16;
    __shared__ double scoef[kCoefN];
    __shared__ int32_t sh_cnt;
    // the chains' tokens, lengths and evidence classes, staged in one round
    // trip (the tokens when they fit)
    constexpr int kChainLds = 2048;
    __shared__ int32_t ctok[kChainLds];
    __shared__ int32_t cfol[kChainLds];   // follower counts (0: a copied token)
    __shared__ int32_t clen[SPEC_MAX_FOREST];
    __shared__ int8_t cev[SPEC_MAX_FOREST];
    const int P_ = A.P, Kc = A.Kc, cmax = A.c_max;
    const int nd = 1 + P_ * Kc;
    const int64_t q0 = (int64_t)r * (P_ + 1);
    const bool staged = (int64_t)(P_ + 1) * A.ngram_ld <= kChainLds;
    // the Eq. (6) inputs of the drafter nodes on the first threads (node i on
    // thread i) and the request's own terms, requested now so that the
    // weights do not wait for them after the walk
    float pf_h = 0.5f, pf_s = 0.5f, pf_r = 1.0f, pf_src = 0.5f, pf_ctx = 0.0f, pf_req = 0.0f;
    if (P.scored) {
        pf_src = P.sc.p_src[r];
        pf_ctx = P.sc.psi_ctx[r];
        pf_req = P.sc.b_req[r];
        if (t >= 1 && t < nd) {
            const int p = (t - 1) / Kc + 1, k = (t - 1) % Kc;
            pf_h = P.sc.h[(int64_t)r * P_ + p - 1];
            pf_s = P.sc.sigma[(int64_t)r * P_ + p - 1];
            if (k > 0) pf_r = P.sc.r_share[((int64_t)r * P_ + p - 1) * Kc + k];
        }
    }
    if (P.scored && t < kCoefN) {
        const spec_tree_scores& S = P.sc;
        scoef[t] = t < kCoefAg ? S.w_bucket[t]
                 : t < kCoefCo ? S.w_agreed[(t - kCoefAg) >> 1][(t - kCoefAg) & 1]
                 : t < kCoefPsi ? S.w_contra[(t - kCoefCo) >> 1][(t - kCoefCo) & 1]
                 : S.psi_depth[t - kCoefPsi];
    }
    for (int i = t; i <= P_; i += kTreeBlock) {
        clen[i] = A.ngram_len[q0 + i];
        cev[i] = (int8_t)(P.scored ? evidence_of(P.sc.ngram_feat + 4 * (q0 + i)) : 0);
    }
    if (staged)
        for (int i = t; i < (P_ + 1) * A.ngram_ld; i += kTreeBlock) {
            ctok[i] = A.ngram_draft[q0 * A.ngram_ld + i];
            cfol[i] = A.ngram_follow ? A.ngram_follow[q0 * A.ngram_ld + i] : 0;
        }
    // the drafter nodes: parent, token, depth, kind; n-gram nodes above,
    // bucket, agreeing bucket.  Slots past the node count hold parent -2.
    int rpar[NS], rtok[NS], rdep[NS], rkind[NS], rabove[NS], rbucket[NS], ragree[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int i = s * kWave + lane;
        rpar[s] = -2; rtok[s] = -2; rdep[s] = 0; rkind[s] = 0; rabove[s] = 0; rbucket[s] = -1; ragree[s] = -1;
        if (i == 0) {
            rpar[s] = -1; rtok[s] = -1;
        } else if (i < nd) {
            const int p = (i - 1) / Kc + 1, k = (i - 1) % Kc;
            rtok[s] = A.block[((int64_t)r * P_ + (p - 1)) * Kc + k];
            rpar[s] = (p == 1) ? 0 : 1 + (p - 2) * Kc;
            rdep[s] = p;
            rkind[s] = k == 0 ? 1 : 2;
        }
    }
    // With the chains on the lanes and their tokens in LDS, all chains walk
    // together in one parallel pass (below); otherwise, and for the largest
    // forests (whose register slots leave no room for both walks), one chain
    // after another.  The parallel walk's set-up and its drafter nodes (whose
    // tokens it reads) go in before the first barrier.
    const bool parallel_walk = NS <= 8 && P_ < kWave && staged;
    uint32_t flags = 0;
    if (parallel_walk) {
        if (wid == 0) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int n = s * kWave + lane;
                if (n < nd) {
                    ftok[n] = rtok[s];
                    fpar[n] = rpar[s];
                    fdep[n] = rdep[s];
                    fkind[n] = (uint8_t)rkind[s];
                    fabove[n] = 0;
                    fbucket[n] = -1;
                    fagree[n] = -1;
                }
            }
        }
        walk_parallel_init(A, P_, nd, q0, kTreeBlock, reinterpret_cast<wi32*>(fQ), reinterpret_cast<wi32*>(fden),
                           flags);
    }
    __syncthreads();
    // n-gram chains from the anchor (s = 0) and each pick s
    int cntr = nd;
    // the chains' lengths and evidence classes on the lanes (chain sc on lane
    // sc) when there are at most 64 chains
    const bool lane_chains = P_ < kWave;
    const int lglen = lane_chains && lane <= P_ ? clen[lane] : 0;
    const int lev = lane_chains && lane <= P_ ? (int)cev[lane] : 0;
    // with the chains on the lanes, the walk visits only those with tokens
    // (an empty chain adds nothing and passes no node)
    uint64_t live = __builtin_amdgcn_ballot_w64(lglen > 0);
    if (__builtin_amdgcn_ballot_w64(lglen < 0)) flags |= SPEC_FLAG_BAD_LENGTH;
    if (parallel_walk) {
      cntr = walk_parallel(A, P_, Kc, nd, cmax, kTreeBlock, cev, ctok, cfol, ftok, fpar, fdep, fkind, fabove,
                           fbucket, fagree, reinterpret_cast<wi32*>(fw), reinterpret_cast<wi32*>(fQ),
                           reinterpret_cast<wi32*>(fden));
    } else {
    // One chain after another on wave 0.  The walk's state (current node, its
    // depth, kind and n-gram count, the node count) is wave-uniform.  A chain
    // first descends through existing nodes while its tokens match (the
    // lowest-index matching child each time) and then appends the rest of its
    // tokens as a new path.
    for (int it = 0; wid == 0 && it <= P_; ++it) {
        int sc = it;
        if (lane_chains) {
            if (!live) break;
            sc = (int)__builtin_ctzll(live);
            live &= live - 1;
        }
        const int64_t q = q0 + sc;
        int glen = lane_chains ? __builtin_amdgcn_readlane(lglen, sc) : clen[sc];
        if (glen < 0 || glen > A.ngram_ld) { flags |= SPEC_FLAG_BAD_LENGTH; glen = glen < 0 ? 0 : A.ngram_ld; }
        if (glen == 0) continue;   // nothing to walk or add
        const int ev = lane_chains ? __builtin_amdgcn_readlane(lev, sc) : (int)cev[sc];
        // token i of the chain and its follower count (0: a copied token),
        // read from LDS or from global memory through pointers of their own
        // address space (a pointer that may be either compiles to flat loads,
        // which wait for every outstanding access)
        const int32_t* lsrc = ctok + (int64_t)sc * A.ngram_ld;
        const int32_t* lfol = cfol + (int64_t)sc * A.ngram_ld;
        const gi32_ptr gsrc = (gi32_ptr)(A.ngram_draft + q * A.ngram_ld);
        const gi32_ptr gfol = (gi32_ptr)(A.ngram_follow ? A.ngram_follow + q * A.ngram_ld : nullptr);
        auto tok_at = [&](int i) -> int32_t { return staged ? lsrc[i] : gsrc[i]; };
        auto fol_at = [&](int i) -> int32_t { return staged ? lfol[i] : (gfol ? gfol[i] : 0); };
        // a token's bucket base: 4 x the copy's evidence class, or 32 + 4 x the
        // class of its follower count
        auto base_of = [&](int32_t fc) { return fc > 0 ? 32 + 4 * follower_class(fc) : 4 * ev; };
        int cur = (sc == 0) ? 0 : 1 + (sc - 1) * Kc;   // a drafter node (< nd <= 1024)
        int cdep = 0, ckind = 0, cabove = 0;
        auto read_cur = [&]() {   // cur's depth, kind and n-gram count, from its lane
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (s == (cur >> 6)) {
                    cdep = __builtin_amdgcn_readlane(rdep[s], cur & 63);
                    ckind = __builtin_amdgcn_readlane(rkind[s], cur & 63);
                    cabove = __builtin_amdgcn_readlane(rabove[s], cur & 63);
                }
        };
        read_cur();
        int ctk = lane < glen ? tok_at(lane) : -1;   // the chain's first 64 tokens and their bucket bases
        int cfb = base_of(lane < glen ? fol_at(lane) : 0);
        int t = 0;
        bool tail = false;
        if (glen <= kWave) {
            // A node can only be the descent's t-th step if it sits at depth
            // d0 + 1 + t and holds token t; such nodes key on their parent, the
            // others never match.  The descent then costs one ballot per token.
            const int d0 = cdep;
            const int geff = glen < A.depth_max - d0 ? glen : A.depth_max - d0;
            int key[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                key[s] = -2;
                if (s * kWave < cntr) {
                    const int tn = rdep[s] - d0 - 1;
                    const int tkn = __shfl(ctk, tn & 63, kWave);
                    key[s] = (tn >= 0 && tn < geff && rtok[s] == tkn) ? rpar[s] : -2;
                }
            }
            uint64_t pm[NS];   // the nodes passed, as lane masks per slot
#pragma unroll
            for (int s = 0; s < NS; ++s) pm[s] = 0;
            if (cntr <= kWave) {
                // every node in slot 0: one compare, one ballot per token
                while (t < geff) {
                    const uint64_t bal = __builtin_amdgcn_ballot_w64(key[0] == cur);
                    if (!bal) break;
                    cur = (int)__builtin_ctzll(bal);
                    pm[0] |= 1ull << cur;
                    ++t;
                }
            }
            while (t < geff && cntr > kWave) {
                int nxt = -1;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (nxt < 0 && s * kWave < cntr) {
                        const uint64_t bal = __builtin_amdgcn_ballot_w64(key[s] == cur);
                        if (bal) {
                            const int l = (int)__builtin_ctzll(bal);
                            pm[s] |= 1ull << l;
                            nxt = s * kWave + l;
                        }
                    }
                }
                if (nxt < 0) break;
                cur = nxt;
                ++t;
            }
            // every node passed records the agreement: the proposal's bucket
            // counts the n-gram nodes above the node, its own n-gram count
            if (t > 0) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int tn = rdep[s] - d0 - 1;   // the chain token that passed this node
                    const int tb = __shfl(cfb, tn & 63, kWave);
                    if ((pm[s] >> lane) & 1ull) {
                        const int b = tb + (rabove[s] < 3 ? rabove[s] : 3);
                        if ((rkind[s] & 3) != 3 && b > ragree[s]) ragree[s] = b;
                        rkind[s] |= 4;
                    }
                }
                read_cur();
            }
            tail = t < geff && cntr < cmax;
        } else {
            // chains longer than a wave: one token per step
            for (; t < glen; ++t) {
                if (cdep + 1 > A.depth_max) break;
                if (t && (t & 63) == 0) {   // the next 64
                    ctk = t + lane < glen ? tok_at(t + lane) : -1;
                    cfb = base_of(t + lane < glen ? fol_at(t + lane) : 0);
                }
                const int tk = __builtin_amdgcn_readlane(ctk, t & 63);
                const int up = cabove + ((ckind & 3) == 3);   // n-gram nodes above a child of cur
                const int bucket = __builtin_amdgcn_readlane(cfb, t & 63) + (up < 3 ? up : 3);
                int found = -1, fk = 0, fd = 0, fa = 0;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (found < 0 && s * kWave < cntr) {
                        const uint64_t bal = __builtin_amdgcn_ballot_w64(rpar[s] == cur && rtok[s] == tk);
                        if (bal) {
                            const int l = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(bal));
                            found = s * kWave + l;
                            fk = __builtin_amdgcn_readlane(rkind[s], l);
                            fd = __builtin_amdgcn_readlane(rdep[s], l);
                            fa = __builtin_amdgcn_readlane(rabove[s], l);
                            // the match's own lane records the agreement (selects,
                            // not a branch, so the walk's state stays scalar)
                            const bool me = lane == l;
                            ragree[s] = (me && (fk & 3) != 3 && bucket > ragree[s]) ? bucket : ragree[s];
                            rkind[s] = me ? (fk | 4) : rkind[s];
                        }
                    }
                }
                if (found < 0) {
                    tail = cntr < cmax;
                    break;
                }
                cur = found;
                cdep = fd;
                ckind = fk | 4;
                cabove = fa;
            }
        }
        if (tail) {
            // a new node has no children yet, so every later token of the
            // chain becomes a new node too: node cntr + i is token t + i
            // (the chain's length, the depth limit and c_max bound them)
            const int up = cabove + ((ckind & 3) == 3);   // n-gram nodes above a child of cur
            int rem = glen - t;
            rem = rem < A.depth_max - cdep ? rem : A.depth_max - cdep;
            rem = rem < cmax - cntr ? rem : cmax - cntr;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int n = s * kWave + lane, i = n - cntr;
                if (i >= 0 && i < rem) {
                    const int ui = up + i;
                    rtok[s] = tok_at(t + i);
                    rpar[s] = i == 0 ? cur : n - 1;
                    rdep[s] = cdep + 1 + i;
                    rkind[s] = 3;
                    rabove[s] = ui < 127 ? ui : 127;
                    rbucket[s] = base_of(fol_at(t + i)) + (ui < 3 ? ui : 3);
                    ragree[s] = -1;
                }
            }
            cntr += rem;
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int n = s * kWave + lane;
        if (wid == 0 && n < cntr) {
            ftok[n] = rtok[s];
            fpar[n] = rpar[s];
            fdep[n] = rdep[s];
            fkind[n] = (uint8_t)rkind[s];
            fabove[n] = (int8_t)rabove[s];
            fbucket[n] = (int8_t)rbucket[s];
            fagree[n] = (int8_t)ragree[s];
        }
    }
    }
    for (int j = t; j < nd; j += kTreeBlock) fcontra[j] = -1;
    if (t == 0) sh_cnt = cntr;
    __syncthreads();
    const int cnt = sh_cnt;
    // weights: given by candidate index, or exp of the Eq. (6) scores (none = 1)
    const float* wn = A.w_node + (int64_t)r * cmax;
    const float* wz = A.w_none + (int64_t)r * cmax;
    if (P.scored) {
        // contradictions: an n-gram node whose parent is the anchor or a pick
        // hands its evidence class to the drafter nodes of the next position
        // (those that share its parent) that hold another token; the largest
        // class counts
        for (int c = nd + t; c < cnt; c += kTreeBlock) {
            const int pn = fpar[c];
            const int pos = pn == 0 ? 1 : ((pn < nd && (pn - 1) % Kc == 0) ? fdep[pn] + 1 : 0);
            if (pos >= 1 && pos <= P_) {
                const int cls = (fbucket[c] & 31) / 4;   // the evidence class, of either kind
                const int32_t tk = ftok[c];
                for (int k = 0; k < Kc; ++k) {
                    const int j = 1 + (pos - 1) * Kc + k;
                    if (ftok[j] != tk) atomicMax(&fcontra[j], cls);
                }
            }
        }
        __syncthreads();
        const spec_tree_scores& S = P.sc;
        const double lps = logit_prob((double)pf_src);
        const double plus = lps > 0.0 ? lps : 0.0;
        const double pc = (double)pf_ctx, br = (double)pf_req;
        for (int j = t; j < cnt; j += kTreeBlock) {
            const bool pre = j < kTreeBlock;   // node j is on thread j: its inputs are in registers
            double sj = 0.0;
            const int kind = fkind[j] & 3;
            if (j == 0) {
                fw[j] = 0.0;
                continue;
            }
            if (kind == 3) {
                sj = lps + scoef[fbucket[j]] + pc + br;
            } else {
                const int p = fdep[j], k = (j - 1) % Kc, ps = kind == 1 ? 0 : 1;
                const double lh = logit_prob((double)(pre ? pf_h : S.h[(int64_t)r * P_ + p - 1]));
                const double ls = logit_prob((double)(pre ? pf_s : S.sigma[(int64_t)r * P_ + p - 1]));
                const double psi = pc + scoef[kCoefPsi + (p < 15 ? p : 15)];
                if (kind == 1) {
                    sj = S.a[0] + S.a[1] * lh + S.a[2] * ls + psi + br;
                } else {
                    const double rr = clamp_prob((double)(pre ? pf_r : S.r_share[((int64_t)r * P_ + p - 1) * Kc + k]));
                    sj = S.a[3] + S.a[4] * log(rr) + S.a[5] * lh + S.a[6] * ls + psi + br;
                }
                if (fagree[j] >= 0) sj += plus + scoef[kCoefAg + 2 * fagree[j] + ps];
                const int contra = fcontra[j];
                if (contra >= 0) sj += -plus + scoef[kCoefCo + 2 * contra + ps];
            }
            fw[j] = exp(sj);
        }
    } else {
        for (int j = t; j < cnt; j += kTreeBlock) fw[j] = (double)wn[j];
    }
    __syncthreads();
    // denominators of the Eq. (6) form: none + the children's weights (index
    // order), then Q = the parent's Q times w / den along every path (index
    // order, so a parent is done before its children)
    if (cnt <= kWave) {
      if (wid == 0) {
        // one node per lane.  Each node's children as a lane mask (index
        // order); a parent adds its lowest remaining child per round, so the
        // sums keep index order and take as many rounds as the widest node
        // has children.  Q then goes one depth level per round (a child is one
        // level below its parent).
        const bool mine = lane < cnt;
        const int pj = mine ? fpar[lane] : -2;
        const int dj = mine ? fdep[lane] : -1;
        const double wj = mine ? fw[lane] : 0.0;
        // (one wave: its LDS operations run in order; the fences keep the
        // compiler from moving the zeroing, the ors and the read past each other)
        fkids[lane] = 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (mine && lane > 0) atomicOr(&fkids[pj], 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        uint64_t kids = mine ? fkids[lane] : 0;
        double den = P.scored ? 1.0 : (mine ? (double)wz[lane] : 0.0);
        while (__builtin_amdgcn_ballot_w64(kids != 0)) {
            const double wc = shfl_f64(wj, kids ? (int)__builtin_ctzll(kids) : 0);
            den = kids ? den + wc : den;
            kids &= kids - 1;
        }
        const double ratio = wj / shfl_f64(den, pj < 0 ? 0 : pj);
        // Q four levels per round: a node k levels below the round's first
        // depth d takes Q of its ancestor at depth d - 1 (final since the last
        // round) and multiplies in the ratios down its path, top first: the
        // parent-times-ratio product in the same order
        const int a1 = pj < 0 ? 0 : pj;
        const int a2 = __shfl(a1, a1, kWave), a3 = __shfl(a1, a2, kWave), a4 = __shfl(a1, a3, kWave);
        const double r1 = shfl_f64(ratio, a1), r2 = shfl_f64(ratio, a2), r3 = shfl_f64(ratio, a3);
        double q = 1.0;
        for (int d = 1; __builtin_amdgcn_ballot_w64(dj >= d); d += 4) {
            const int k = dj - d;
            const double qa = shfl_f64(q, k <= 0 ? a1 : (k == 1 ? a2 : (k == 2 ? a3 : a4)));
            double v = qa;
            if (k >= 3) v = v * r3;
            if (k >= 2) v = v * r2;
            if (k >= 1) v = v * r1;
            v = v * ratio;
            q = (k >= 0 && k < 4) ? v : q;
        }
        if (mine) {
            fden[lane] = den;
            fQ[lane] = q;
            fsel[lane] = 0;
        }
      }
    } else {
        for (int p = t; p < cnt; p += kTreeBlock) {
            double den = P.scored ? 1.0 : (double)wz[p];
            for (int c = 1; c < cnt; ++c)
                if (fpar[c] == p) den += fw[c];
            fden[p] = den;
            fsel[p] = 0;
        }
        __syncthreads();
        if (t == 0) {
            fQ[0] = 1.0;
            for (int j = 1; j < cnt; ++j) fQ[j] = fQ[fpar[j]] * (fw[j] / fden[fpar[j]]);
        }
    }
    __syncthreads();
    tree_rows(A, r, lane, cnt, flags, ftok, fpar, fQ, fsel);
}

// Rows from a forest the caller built ([AS] Section 3.1): one wave per
// request.  Node j's path probability is its parent's times q_j (fp64, in
// index order, parents first); the rows are then chosen and laid out as in
// the tree build.  A parent outside [0, j) or a q outside [0, 1] breaks the
// forest: the request is flagged and keeps the anchor alone.
__global__ __launch_bounds__(kWave) void k_tree_forest(spec_tree_alloc A)
{
    const int r = blockIdx.x, lane = threadIdx.x;
    __shared__ int32_t ftok[SPEC_MAX_FOREST];
    __shared__ int32_t fpar[SPEC_MAX_FOREST];
    __shared__ float fq[SPEC_MAX_FOREST];
    __shared__ double fQ[SPEC_MAX_FOREST];
    __shared__ uint8_t fsel[SPEC_MAX_FOREST];
    const int cmax = A.c_max;
    const int64_t o = (int64_t)r * cmax;
    uint32_t flags = 0;
    int n = A.forest_n[r];
    if (n < 1 || n > cmax) {
        flags |= SPEC_FLAG_BAD_LENGTH;
        n = n < 1 ? 1 : cmax;
    }
    bool bad = false;
    for (int j = lane; j < n; j += kWave) {
        const int32_t tk = A.forest_token[o + j];
        const int32_t p = A.forest_parent[o + j];
        const float q = A.forest_q[o + j];
        ftok[j] = tk;
        fpar[j] = j == 0 ? -1 : p;
        fq[j] = q;
        fsel[j] = 0;
        bad |= j > 0 && (p < 0 || p >= j || !(q >= 0.0f && q <= 1.0f));
    }
    if (__ballot(bad)) {
        flags |= SPEC_FLAG_BAD_FOREST;
        n = 1;
    }
    __syncthreads();
    // Q in batches of 64 nodes, node base + l on lane l: a parent in an
    // earlier batch is read from LDS, one in the same batch from its lane, in
    // index order so that it is final when its children read it
    for (int base = 0; base < n; base += kWave) {
        const int j = base + lane;
        const bool mine = j < n;
        const int p = mine ? fpar[j] : -1;
        const double qj = mine ? (double)fq[j] : 0.0;
        double Qv = j == 0 ? 1.0 : ((mine && p < base) ? fQ[p] * qj : 0.0);
        const int hi = n - base < kWave ? n - base : kWave;
        for (int l = 0; l < hi; ++l) {
            const int pl = __builtin_amdgcn_readlane(p, l);
            if (pl >= base) {   // wave-uniform
                const double qp = readlane_f64(Qv, pl - base);
                Qv = lane == l ? qp * qj : Qv;
            }
        }
        if (mine) fQ[j] = Qv;
        __syncthreads();
    }
    tree_rows(A, r, lane, n, flags, ftok, fpar, fQ, fsel);
}

__global__ __launch_bounds__(kAllocBlock) void k_rows_scan(const int32_t* n_rows, int bs, int64_t* row_base, int32_t* total_rows)
{
    const int per = (bs + kAllocBlock - 1) / kAllocBlock;
    const int r0 = threadIdx.x * per;
    int64_t local = 0;
    for (int r = r0; r < r0 + per && r < bs; ++r) local += n_rows[r];
    int64_t total;
    int64_t base = block_exclusive_i64(local, &total);
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        row_base[r] = base;
        base += n_rows[r];
    }
    if (threadIdx.x == 0) total_rows[0] = (int32_t)total;
}

}  // namespace spec

using namespace spec;

size_t spec_alloc_ws(const spec_alloc_args* a)
{
    if (a->mode != SPEC_ALLOC_CHAIN) return 0;
    return align256((size_t)a->chain.bs * a->chain.ld * sizeof(uint64_t));   // ranking keys
}

int spec_alloc_launch(const spec_alloc_args* a, hipStream_t st)
{
    if (a->mode == SPEC_ALLOC_CHAIN) {
        SelectParams P;
        P.a = a->chain;
        P.keys = (uint64_t*)a->workspace;
        const int grid = (a->chain.bs + kSlotReqs - 1) / kSlotReqs;
        hipLaunchKernelGGL(k_alloc_slots, dim3(grid), dim3(kSlotBlock), 0, st, P);
        hipLaunchKernelGGL(k_alloc_topk, dim3(1), dim3(kAllocBlock), 0, st, P);
    } else {
        TreeBuildParams P;
        P.a = a->tree;
        P.scored = a->tree.scores != nullptr;
        if (P.scored) P.sc = *a->tree.scores;
        else std::memset(&P.sc, 0, sizeof(P.sc));
        const int c = a->tree.c_max;
        const dim3 g(a->tree.bs), b(kTreeBlock);
        if (a->tree.forest_token) hipLaunchKernelGGL(k_tree_forest, g, dim3(kWave), 0, st, a->tree);
        else if (c <= 64) hipLaunchKernelGGL(k_tree<1>, g, b, 0, st, P);
        else if (c <= 128) hipLaunchKernelGGL(k_tree<2>, g, b, 0, st, P);
        else if (c <= 256) hipLaunchKernelGGL(k_tree<4>, g, b, 0, st, P);
        else if (c <= 512) hipLaunchKernelGGL(k_tree<8>, g, b, 0, st, P);
        else hipLaunchKernelGGL(k_tree<16>, g, b, 0, st, P);
        hipLaunchKernelGGL(k_rows_scan, dim3(1), dim3(kAllocBlock), 0, st, a->tree.n_rows, a->tree.bs, a->tree.row_base,
                           a->tree.total_rows);
    }
    return spec_record_hip_error(hipGetLastError());
}
