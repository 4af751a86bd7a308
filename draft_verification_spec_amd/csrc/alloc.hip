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
//   k_tree    : one wave per request builds the candidate forest in LDS
//               (drafter block + n-gram chains), the acceptance estimates of
//               the Eq. (6) form, the path products Q, the best-first top
//               rows_cap-1 (Proposition 1) and the depth-first layout.
//   k_rows_scan: exclusive prefix sum of the rows per request.
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

// Eq. (1) logit of position k (1-based); `lnm` = ln(min(max(m,1), m_cap) / m_ref).
__device__ __forceinline__ double est_logit(const spec_estimator& e, int k, int n, int a, double lnm)
{
    const bool first = (k == 1);
    double z = (double)e.beta[(k <= 15 ? k : 15) - 1] +
               (double)(first ? e.w_first : e.w_rest) * ((double)n - (double)e.n_ref) + (double)e.delta * (double)a;
    if ((double)n >= (double)e.n_full)
        z += (double)(first ? e.l_first : e.l_rest) + (double)(first ? e.k_first : e.k_rest) * lnm;
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
    const int rl = A.ngram_len[r];
    const int gcap = A.ngram_ld < ld ? A.ngram_ld : ld;
    const int glen = rl < 0 ? 0 : (rl > gcap ? gcap : rl);
    const int n = A.ngram_feat[4 * (int64_t)r + 0];
    const int am = A.ngram_feat[4 * (int64_t)r + 1];
    double mm = (double)A.ngram_feat[4 * (int64_t)r + 2];
    mm = mm < 1.0 ? 1.0 : (mm > (double)A.est.m_cap ? (double)A.est.m_cap : mm);
    const double lnm = ((double)n >= (double)A.est.n_full) ? log(mm / (double)A.est.m_ref) : 0.0;
    const bool mpm = !A.model_point_mass || A.model_point_mass[r];
    const int k = lane;
    int32_t td = -1, tg = -1;
    double h = 0.0, c = 0.0;
    if (k < K) {
        td = A.model_tokens[(int64_t)r * K + k];
        const double cv = (double)A.model_conf[(int64_t)r * K + k];
        c = A.conf_is_logit ? sigm(cv) : cv;
    }
    if (k < gcap) tg = A.ngram_draft[(int64_t)r * A.ngram_ld + k];
    if (k < glen) h = sigm(est_logit(A.est, k + 1, n, am, lnm));
    const bool mismatch = __ballot(k < K && td != tg) != 0;
    // chain values (Eq. (3)) from the running products
    const double lam = (double)A.lambda;
    double sg = 1.0, sd = 1.0, vg = 0.0, vd = 0.0;
    for (int q = 0; q < glen; ++q) {
        sg *= lane_value(h, q);
        vg += sg > lam ? sg - lam : 0.0;
    }
    for (int q = 0; q < K; ++q) {
        sd *= lane_value(c, q);
        vd += sd > lam ? sd - lam : 0.0;
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
    // survivals of the chosen chain; lane k keeps S_k
    sg = 1.0;
    sd = 1.0;
    double prev = 1.0, mine = 0.0;
    for (int q = 0; q < len; ++q) {
        const double hq = (q < glen) ? lane_value(h, q) : 0.0;
        if (q < glen) sg *= hq;
        if (q < K) sd *= lane_value(c, q);
        double S;
        if (use == SPEC_SRC_MODEL) S = sd;
        else if (use == SPEC_SRC_NGRAM) S = sg;
        else if (use == SPEC_SRC_MERGED) S = (q < K) ? (sg > sd ? sg : sd) : prev * hq;
        else S = (q < K) ? sd : prev * hq;
        prev = S;
        if (lane == q) mine = S;
    }
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

__device__ int64_t block_exclusive_i64(int64_t v, int64_t* total)
{
    __shared__ int64_t sh[32];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    const int nw = (int)(blockDim.x / kWave);
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

// Exclusive prefix over the workgroup of 32-bit counts; *total gets the sum.
__device__ uint32_t block_exclusive_u32(uint32_t v, uint32_t* total)
{
    __shared__ uint32_t sh[32];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    const int nw = (int)(blockDim.x / kWave);
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

// The exact budget-th largest ranking key by an 8-bit radix select over the
// survival and position bytes (stopping as soon as the boundary bucket is
// taken whole), the request bits by one ordered scan, then each request's
// verified prefix and the row bases.  One workgroup.
__global__ __launch_bounds__(kAllocBlock) void k_alloc_topk(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int bs = A.bs, ld = A.ld;
    const int64_t N = (int64_t)bs * ld;
    __shared__ uint64_t lkeys[kLdsKeys];
    __shared__ uint32_t hist[2][256];
    __shared__ uint64_t sh_prefix, sh_min;
    __shared__ int64_t sh_rem, sh_valid;
    __shared__ int sh_done;
    const bool in_lds = N <= kLdsKeys;
    uint64_t* keys = in_lds ? lkeys : P.keys;
    const int wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) { sh_prefix = 0; sh_valid = 0; sh_done = 0; sh_min = ~0ull; }
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
    const int64_t take = (A.budget < sh_valid) ? A.budget : sh_valid;
    uint64_t theta = ~0ull;  // nothing selected
    if (take > 0) {
        if (threadIdx.x == 0) sh_rem = take;
        uint64_t mask = 0;
        for (int i = threadIdx.x; i < 256; i += kAllocBlock) hist[0][i] = 0;
        __syncthreads();
        for (int shift = 56, hb = 0; shift >= 0; shift -= 8, hb ^= 1) {
            // the histogram of this pass was cleared during the previous one
            uint32_t* H = hist[hb];
            const uint64_t pre = sh_prefix;
            const int64_t rounds = (N + kAllocBlock - 1) / kAllocBlock;
            for (int64_t u = 0; u < rounds; ++u) {
                const int64_t i = threadIdx.x + u * kAllocBlock;
                const uint64_t k = i < N ? keys[i] : 0ull;
                hist_add(H, k != 0 && (k & mask) == pre, (int)((k >> shift) & 255u));
            }
            for (int i = threadIdx.x; i < 256; i += kAllocBlock) hist[hb ^ 1][i] = 0;
            __syncthreads();
            if (wid == 0) {
                // lane l owns digits 255-4l .. 252-4l (descending); suffix counts from the top
                uint32_t c4[4];
                uint32_t own = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) { c4[j] = H[255 - 4 * lane - j]; own += c4[j]; }
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
        theta = sh_prefix;
        if (sh_done && mask != ~0ull) {
            uint64_t mn = ~0ull;
            for (int64_t i = threadIdx.x; i < N; i += kAllocBlock) {
                const uint64_t k = keys[i];
                if (k != 0 && (k & mask) == theta && k < mn) mn = k;
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                const uint64_t v = __shfl_xor(mn, o, kWave);
                mn = v < mn ? v : mn;
            }
            if (lane == 0) atomicMin((unsigned long long*)&sh_min, (unsigned long long)mn);
            __syncthreads();
            theta = sh_min;
        }
    }
    // verified prefix per request, row bases over (alloc + 1)
    const int per = (bs + (int)blockDim.x - 1) / (int)blockDim.x;
    const int r0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < SPEC_MAX_DRAFT; ++k) {
            if (k < ld) {
                const uint64_t key = keys[(int64_t)r * ld + k];
                cnt += (key != 0 && key >= theta);
            }
        }
        A.alloc_len[r] = cnt;
        local += cnt + 1;
    }
    uint32_t total;
    int64_t base = block_exclusive_u32(local, &total);
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        A.row_base[r] = base;
        base += A.alloc_len[r] + 1;
    }
    if (threadIdx.x == 0) A.total_rows[0] = (int32_t)total;
}

// ---------------------------------------------------------------------------
// trees
// ---------------------------------------------------------------------------

struct TreeBuildParams {
    spec_tree_alloc a;
};

__global__ __launch_bounds__(kWave) void k_tree(TreeBuildParams P)
{
    const spec_tree_alloc& A = P.a;
    const int r = blockIdx.x, lane = threadIdx.x;
    __shared__ int32_t ftok[SPEC_MAX_FOREST];
    __shared__ int32_t fpar[SPEC_MAX_FOREST];
    __shared__ int32_t fdep[SPEC_MAX_FOREST];
    __shared__ double fden[SPEC_MAX_FOREST];
    __shared__ double fQ[SPEC_MAX_FOREST];
    __shared__ uint8_t fsel[SPEC_MAX_FOREST];
    __shared__ int32_t sh_cnt, sh_cur;
    const int P_ = A.P, Kc = A.Kc, cmax = A.c_max;
    const int nd = 1 + P_ * Kc;
    for (int i = lane; i < nd; i += kWave) {
        if (i == 0) { ftok[0] = -1; fpar[0] = -1; fdep[0] = 0; }
        else {
            const int p = (i - 1) / Kc + 1, k = (i - 1) % Kc;
            ftok[i] = A.block[((int64_t)r * P_ + (p - 1)) * Kc + k];
            fpar[i] = (p == 1) ? 0 : 1 + (p - 2) * Kc;
            fdep[i] = p;
        }
    }
    if (lane == 0) sh_cnt = nd;
    __syncthreads();
    // n-gram chains from the anchor (s = 0) and each pick s
    uint32_t flags = 0;
    for (int s = 0; s <= P_; ++s) {
        const int64_t q = (int64_t)r * (P_ + 1) + s;
        int glen = A.ngram_len[q];
        if (glen < 0 || glen > A.ngram_ld) { flags |= SPEC_FLAG_BAD_LENGTH; glen = glen < 0 ? 0 : A.ngram_ld; }
        if (lane == 0) sh_cur = (s == 0) ? 0 : 1 + (s - 1) * Kc;
        __syncthreads();
        for (int t = 0; t < glen; ++t) {
            const int cur = sh_cur;
            if (fdep[cur] + 1 > A.depth_max) break;
            const int32_t tk = A.ngram_draft[q * A.ngram_ld + t];
            const int cnt = sh_cnt;
            int found = -1;
            for (int base = 1; base < cnt && found < 0; base += kWave) {
                const int c = base + lane;
                const bool hit = c < cnt && fpar[c] == cur && ftok[c] == tk;
                const uint64_t bal = __ballot(hit);
                if (bal) found = base + (int)__builtin_ctzll(bal);
            }
            if (found < 0 && cnt >= cmax) break;
            if (lane == 0) {
                if (found >= 0) sh_cur = found;
                else {
                    ftok[cnt] = tk; fpar[cnt] = cur; fdep[cnt] = fdep[cur] + 1;
                    sh_cnt = cnt + 1;
                    sh_cur = cnt;
                }
            }
            __syncthreads();
        }
        __syncthreads();
    }
    const int cnt = sh_cnt;
    // denominators of the Eq. (6) form: w_none[p] + sum of the children's weights (index order)
    const float* wn = A.w_node + (int64_t)r * cmax;
    const float* wz = A.w_none + (int64_t)r * cmax;
    for (int p = lane; p < cnt; p += kWave) {
        double den = (double)wz[p];
        for (int c = 1; c < cnt; ++c)
            if (fpar[c] == p) den += (double)wn[c];
        fden[p] = den;
        fsel[p] = 0;
    }
    __syncthreads();
    if (lane == 0) {
        fQ[0] = 1.0;
        for (int j = 1; j < cnt; ++j) fQ[j] = fQ[fpar[j]] * ((double)wn[j] / fden[fpar[j]]);
    }
    __syncthreads();
    // best-first: rank by (fp32 Q desc, index asc); keep rank < rows_cap - 1
    const int keep = A.rows_cap - 1;
    for (int j = 1 + lane; j < cnt; j += kWave) {
        const uint64_t kj = ((uint64_t)__float_as_uint((float)fQ[j]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
        int rank = 0;
        for (int i = 1; i < cnt; ++i) {
            const uint64_t ki = ((uint64_t)__float_as_uint((float)fQ[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
            rank += ki > kj;
        }
        fsel[j] = rank < keep;
    }
    __syncthreads();
    __shared__ int32_t st_n[SPEC_MAX_ROWS], st_p[SPEC_MAX_ROWS];
    if (lane == 0) {
        fsel[0] = 1;
        // depth-first layout, children in index order
        int sp = 0, row = 0;
        st_n[sp] = 0; st_p[sp] = -1; ++sp;
        int32_t* nt = A.node_token + (int64_t)r * A.rows_cap;
        int32_t* pr = A.parent_row + (int64_t)r * A.rows_cap;
        float* Qo = A.Q + (int64_t)r * A.rows_cap;
        while (sp > 0 && row < A.rows_cap) {
            --sp;
            const int u = st_n[sp];
            nt[row] = (u == 0) ? -1 : ftok[u];
            pr[row] = st_p[sp];
            Qo[row] = (float)fQ[u];
            const int my = row++;
            for (int c = cnt - 1; c >= 1; --c)
                if (fsel[c] && fpar[c] == u && sp < SPEC_MAX_ROWS) { st_n[sp] = c; st_p[sp] = my; ++sp; }
        }
        for (int i = row; i < A.rows_cap; ++i) { nt[i] = -1; pr[i] = -1; Qo[i] = 0.0f; }
        A.n_rows[r] = row;
        A.forest_count[r] = cnt;
        A.out_flags[r] = flags;
    }
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
        hipLaunchKernelGGL(k_tree, dim3(a->tree.bs), dim3(kWave), 0, st, P);
        hipLaunchKernelGGL(k_rows_scan, dim3(1), dim3(kAllocBlock), 0, st, a->tree.n_rows, a->tree.bs, a->tree.row_base,
                           a->tree.total_rows);
    }
    return spec_record_hip_error(hipGetLastError());
}
