// Verification-budget allocation.
//
// Chains (Hybrid Spark, Algorithm 1 and Sections 4.2-4.4), one launch of one
// 1024-thread workgroup (k_alloc_chain):
//   * every n-gram estimate (Eq. (1)) and model confidence is evaluated in
//     fp64 by its own thread into LDS, next to both chains' tokens (all input
//     is read once, coalesced); then one thread per request forms the
//     survival running products, the chain values of Eq. (3) and the choice
//     (contains rule, value rule with ties to the n-gram chain, or a lossless
//     policy of Appendix H) and leaves the chosen chain's survivals in LDS;
//   * one thread per slot writes the chosen chain and one 64-bit ranking key:
//     fp32(S) bits | (31 - position) | (2^27 - 1 - request), so the largest
//     key is "highest survival, then lower position, then lower request" and
//     keys are unique;
//   * the exact budget-th largest key by an 8-bit radix select over an LDS
//     histogram (the digit is found by a wave-wide suffix scan), stopping as
//     soon as the boundary bucket is taken whole;
//   * each request's verified prefix and the CSR row bases.
// Trees (AdaSpark, Sections 2.2, 3.1, 3.3):
//   k_tree    : one wave per request builds the candidate forest in LDS
//               (drafter block + n-gram chains), the acceptance estimates of
//               the Eq. (6) form, the path products Q, the best-first top
//               rows_cap-1 (Proposition 1) and the depth-first layout.
//   k_rows_scan: exclusive prefix sum of the rows per request.
#include "common.hpp"

namespace spec {

constexpr int kAllocBlock = 1024;
constexpr int kLdsKeys = 4096;          // ranking keys kept in LDS (32 KB); more go to the workspace
constexpr int kLdsVals = 10240;         // fp64 per-slot values kept in LDS (80 KB); more go to the workspace

struct SelectParams {
    spec_chain_alloc a;
    uint64_t* keys;  // workspace fallback: [bs, ld]
    double* vals;    // workspace fallback for the staging area below
};

// Staging area, in 8-byte units per request: ld estimates (later survivals),
// K confidences, the copy-length log term, four int32 words (length state,
// n, a, choice) and the slot tokens of both chains (2 x ld int32).
__host__ __device__ __forceinline__ int64_t vals_count(int64_t bs, int64_t ld, int64_t K) { return bs * (2 * ld + K + 3); }

// length-state word: n-gram length (clamped) | flags
constexpr int kGlMask = 0xFF;
constexpr int kGlMismatch = 1 << 28;   // n-gram and model tokens differ within the first K
constexpr int kGlPointMass = 1 << 29;  // model slots are point masses
constexpr int kGlBadLen = 1 << 30;     // the given n-gram length was out of range

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

// Request r: chain values from its estimates h[0..glen) and confidences
// c[0..K) (the survival running products are left folds, as defined), the
// chain choice, then the chosen chain's survivals written over h (slot k's
// survival replaces h[k] once h[k] has been used).  `gl` is the request's
// length-state word.  Returns (source << 8) | length.
__device__ int select_fold(const spec_chain_alloc& A, int gl, double* h, const double* cc)
{
    const int K = A.K, ld = A.ld;
    const int glen = gl & kGlMask;
    const double lam = (double)A.lambda;
    double sg = 1.0, sd = 1.0, vg = 0.0, vd = 0.0;
    for (int k = 0; k < glen; ++k) {
        sg *= h[k];
        vg += sg > lam ? sg - lam : 0.0;
    }
    for (int k = 0; k < K; ++k) {
        sd *= cc[k];
        vd += sd > lam ? sd - lam : 0.0;
    }
    const bool prefix = glen > K && !(gl & kGlMismatch);
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
    sg = 1.0;
    sd = 1.0;
    double prev = 1.0;
    for (int k = 0; k < ld; ++k) {
        const double hk = (k < glen) ? h[k] : 0.0;
        if (k < glen) sg *= hk;
        if (k < K) sd *= cc[k];
        double S = 0.0;
        if (k < len) {
            if (use == SPEC_SRC_MODEL) S = sd;
            else if (use == SPEC_SRC_NGRAM) S = sg;
            else if (use == SPEC_SRC_MERGED) S = (k < K) ? (sg > sd ? sg : sd) : prev * hk;
            else S = (k < K) ? sd : prev * hk;
            prev = S;
        }
        h[k] = S;
    }
    return (use << 8) | len;
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

// Histogram increment with the lanes that share the first active lane's digit
// folded into one LDS atomic (at the top digits nearly every key agrees).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, int dg)
{
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const int ldg = __shfl(dg, leader, kWave);
    const uint64_t peers = __ballot(active && dg == ldg);
    const int lane = threadIdx.x % kWave;
    if (lane == leader) atomicAdd(&hist[ldg], (uint32_t)__popcll(peers));
    else if (active && dg != ldg) atomicAdd(&hist[dg], 1u);
}

// Chain selection for every request, then the exact budget-th largest key by
// an 8-bit radix select, the verified prefix per request and the row bases.
__global__ __launch_bounds__(kAllocBlock) void k_alloc_chain(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int bs = A.bs, ld = A.ld, K = A.K;
    const int64_t N = (int64_t)bs * ld;
    __shared__ uint64_t lkeys[kLdsKeys];
    __shared__ double lvals[kLdsVals];
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sh_prefix, sh_min;
    __shared__ int64_t sh_rem, sh_valid;
    __shared__ int sh_done;
    uint64_t* keys = (N <= kLdsKeys) ? lkeys : P.keys;
    double* H = (vals_count(bs, ld, K) <= kLdsVals) ? lvals : P.vals;
    double* Cc = H + N;
    double* LNM = Cc + (int64_t)bs * K;
    int32_t* GL = (int32_t*)(LNM + bs);
    int32_t* FN = GL + bs;
    int32_t* FA = FN + bs;
    int32_t* CH = FA + bs;
    int32_t* TD = CH + bs;      // model token per slot
    int32_t* TG = TD + N;       // n-gram token per slot
    const int wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) { sh_prefix = 0; sh_valid = 0; sh_done = 0; sh_min = ~0ull; }
    // 1a. per request: lengths, match features, the copy-length log term
    for (int r = threadIdx.x; r < bs; r += kAllocBlock) {
        const int rl = A.ngram_len[r];
        const int n = A.ngram_feat[4 * (int64_t)r + 0];
        const int am = A.ngram_feat[4 * (int64_t)r + 1];
        double mm = (double)A.ngram_feat[4 * (int64_t)r + 2];
        const bool mpm = !A.model_point_mass || A.model_point_mass[r];
        const int gcap = A.ngram_ld < ld ? A.ngram_ld : ld;
        const int glen = rl < 0 ? 0 : (rl > gcap ? gcap : rl);
        GL[r] = glen | (mpm ? kGlPointMass : 0) | ((rl < 0 || rl > gcap) ? kGlBadLen : 0);
        FN[r] = n;
        FA[r] = am;
        mm = mm < 1.0 ? 1.0 : (mm > (double)A.est.m_cap ? (double)A.est.m_cap : mm);
        LNM[r] = ((double)n >= (double)A.est.n_full) ? log(mm / (double)A.est.m_ref) : 0.0;
    }
    __syncthreads();
    // 1b. per slot: tokens of both chains, the model confidence and the
    // n-gram estimate (fp64), the first-K agreement of the two chains
    for (int64_t i = threadIdx.x; i < N; i += kAllocBlock) {
        const int r = (int)(i / ld), k = (int)(i - (int64_t)r * ld);
        int32_t td = -1, tg = -1;
        double cv = 0.0;
        if (k < K) {
            td = A.model_tokens[(int64_t)r * K + k];
            cv = (double)A.model_conf[(int64_t)r * K + k];
        }
        if (k < A.ngram_ld) tg = A.ngram_draft[(int64_t)r * A.ngram_ld + k];
        const int gl = GL[r];
        const int glen = gl & kGlMask;
        H[i] = (k < glen) ? sigm(est_logit(A.est, k + 1, FN[r], FA[r], LNM[r])) : 0.0;
        if (k < K) Cc[(int64_t)r * K + k] = A.conf_is_logit ? sigm(cv) : cv;
        TD[i] = td;
        TG[i] = tg;
        if (k < K && glen > K && td != tg) atomicOr(&GL[r], kGlMismatch);
    }
    __syncthreads();
    // 1c. one thread per request: values, choice, survivals (over H)
    {
        int64_t valid = 0;
        for (int r = threadIdx.x; r < bs; r += kAllocBlock) {
            const int gl = GL[r];
            const int ch = select_fold(A, gl, H + (int64_t)r * ld, Cc + (int64_t)r * K);
            CH[r] = ch;
            valid += ch & 255;
            A.chain_len[r] = ch & 255;
            A.chain_src[r] = ch >> 8;
            A.out_flags[r] = (gl & kGlBadLen) ? SPEC_FLAG_BAD_LENGTH : 0u;
        }
        valid = wave_sum(valid);
        if (lane == 0) atomicAdd((unsigned long long*)&sh_valid, (unsigned long long)valid);
    }
    __syncthreads();
    // 1d. per-slot outputs and ranking keys
    for (int64_t i = threadIdx.x; i < N; i += kAllocBlock) {
        const int r = (int)(i / ld), k = (int)(i - (int64_t)r * ld);
        const int ch = CH[r], use = ch >> 8, len = ch & 255;
        int32_t tk = -1;
        uint8_t fl = 0;
        const double S = H[i];
        if (k < len) {
            const bool model_slot = use == SPEC_SRC_MODEL || (use == SPEC_SRC_EXTENDED && k < K);
            const bool mpm = (GL[r] & kGlPointMass) != 0;
            tk = (use == SPEC_SRC_MODEL) ? TD[i] : TG[i];
            fl = model_slot ? (mpm ? SPEC_SLOT_POINT_MASS : 0) : (SPEC_SLOT_POINT_MASS | SPEC_SLOT_FROM_NGRAM);
        }
        A.chain_tokens[i] = tk;
        A.slot_flags[i] = fl;
        A.survival[i] = (float)S;
        keys[i] = (k < len) ? (((uint64_t)__float_as_uint((float)S) << 32) | ((uint64_t)(31 - k) << 27) |
                               (uint64_t)(0x7FFFFFF - r))
                            : 0ull;
    }
    __syncthreads();
    const int64_t take = (A.budget < sh_valid) ? A.budget : sh_valid;
    uint64_t theta = ~0ull;  // nothing selected
    if (take > 0) {
        if (threadIdx.x == 0) sh_rem = take;
        uint64_t mask = 0;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = threadIdx.x; i < 256; i += kAllocBlock) hist[i] = 0;
            __syncthreads();
            const uint64_t pre = sh_prefix;
            const int64_t rounds = (N + kAllocBlock - 1) / kAllocBlock;
            for (int64_t u = 0; u < rounds; ++u) {
                const int64_t i = threadIdx.x + u * kAllocBlock;
                const uint64_t k = i < N ? keys[i] : 0ull;
                hist_add(hist, k != 0 && (k & mask) == pre, (int)((k >> shift) & 255u));
            }
            __syncthreads();
            if (wid == 0) {
                // lane l owns digits 255-4l .. 252-4l (descending); suffix counts from the top
                uint32_t c4[4];
                uint32_t own = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) { c4[j] = hist[255 - 4 * lane - j]; own += c4[j]; }
                uint32_t inc = own;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    uint32_t u = __shfl_up(inc, o, kWave);
                    if (lane >= o) inc += u;
                }
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
    // 3. verified prefix per request, row bases over (alloc + 1)
    const int per = (bs + (int)blockDim.x - 1) / (int)blockDim.x;
    const int r0 = threadIdx.x * per;
    int64_t local = 0;
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        int cnt = 0;
        for (int k = 0; k < ld; ++k) {
            const uint64_t key = keys[(int64_t)r * ld + k];
            cnt += (key != 0 && key >= theta);
        }
        A.alloc_len[r] = cnt;
        local += cnt + 1;
    }
    int64_t total;
    int64_t base = block_exclusive_i64(local, &total);
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
    const int64_t N = (int64_t)a->chain.bs * a->chain.ld;
    const int64_t NV = vals_count(a->chain.bs, a->chain.ld, a->chain.K);
    size_t b = 0;
    if (N > kLdsKeys) b += align256((size_t)N * sizeof(uint64_t));
    if (NV > kLdsVals) b += align256((size_t)NV * sizeof(double));
    return b;
}

int spec_alloc_launch(const spec_alloc_args* a, hipStream_t st)
{
    if (a->mode == SPEC_ALLOC_CHAIN) {
        SelectParams P;
        P.a = a->chain;
        const int64_t N = (int64_t)a->chain.bs * a->chain.ld;
        char* ws = (char*)a->workspace;
        P.keys = nullptr;
        if (N > kLdsKeys) {
            P.keys = (uint64_t*)ws;
            ws += align256((size_t)N * sizeof(uint64_t));
        }
        P.vals = (double*)ws;
        hipLaunchKernelGGL(k_alloc_chain, dim3(1), dim3(kAllocBlock), 0, st, P);
    } else {
        TreeBuildParams P;
        P.a = a->tree;
        hipLaunchKernelGGL(k_tree, dim3(a->tree.bs), dim3(kWave), 0, st, P);
        hipLaunchKernelGGL(k_rows_scan, dim3(1), dim3(kAllocBlock), 0, st, a->tree.n_rows, a->tree.bs, a->tree.row_base,
                           a->tree.total_rows);
    }
    return spec_record_hip_error(hipGetLastError());
}
