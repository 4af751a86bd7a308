// Verification-budget allocation.
//
// Chains (Hybrid Spark, Algorithm 1 and Sections 4.2-4.4):
//   k_select  : one thread per request computes the n-gram estimates (Eq. (1)),
//               both survival curves, the chain choice (contains rule, value
//               rule of Eq. (3) with ties to the n-gram chain, or a lossless
//               policy of Appendix H) in fp64, writes the chosen chain to
//               fixed-size buffers and one 64-bit ranking key per slot:
//               fp32(S) bits | (31 - position) | (2^27 - 1 - request), so the
//               largest key is "highest survival, then lower position, then
//               lower request" and keys are unique.
//   k_topk    : one workgroup finds the exact budget-th largest key by an
//               8-bit radix select over LDS histograms, counts each request's
//               verified prefix and writes the CSR row bases.
// Trees (AdaSpark, Sections 2.2, 3.1, 3.3):
//   k_tree    : one wave per request builds the candidate forest in LDS
//               (drafter block + n-gram chains), the acceptance estimates of
//               the Eq. (6) form, the path products Q, the best-first top
//               rows_cap-1 (Proposition 1) and the depth-first layout.
//   k_rows_scan: exclusive prefix sum of the rows per request.
#include "common.hpp"

namespace spec {

constexpr int kLdMax = SPEC_MAX_DRAFT;

struct SelectParams {
    spec_chain_alloc a;
    uint64_t* keys;  // [bs, ld]
};

__device__ __forceinline__ double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

__device__ double est_logit(const spec_estimator& e, int k, int n, int a, int m)
{
    const bool first = (k == 1);
    double z = (double)e.beta[k - 1] + (double)(first ? e.w_first : e.w_rest) * ((double)n - (double)e.n_ref) +
               (double)e.delta * (double)a;
    if ((double)n >= (double)e.n_full) {
        double mm = (double)m;
        if (mm < 1.0) mm = 1.0;
        if (mm > (double)e.m_cap) mm = (double)e.m_cap;
        z += (double)(first ? e.l_first : e.l_rest) + (double)(first ? e.k_first : e.k_rest) * log(mm / (double)e.m_ref);
    }
    return z;
}

__device__ __forceinline__ double chain_value(const double* S, int len, double lam)
{
    double v = 0.0;
    for (int k = 0; k < len; ++k) v += (S[k] > lam) ? (S[k] - lam) : 0.0;
    return v;
}

__global__ __launch_bounds__(64) void k_select(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= A.bs) return;
    const int K = A.K, ld = A.ld;
    uint32_t flags = 0;
    int glen = A.ngram_len[r];
    const int gcap = A.ngram_ld < ld ? A.ngram_ld : ld;
    if (glen < 0 || glen > gcap) { flags |= SPEC_FLAG_BAD_LENGTH; glen = glen < 0 ? 0 : gcap; }
    const int n = A.ngram_feat[4 * (int64_t)r + 0];
    const int am = A.ngram_feat[4 * (int64_t)r + 1];
    const int m = A.ngram_feat[4 * (int64_t)r + 2];
    double h[kLdMax], Sg[kLdMax], Sd[kLdMax];
    double s = 1.0;
    for (int k = 0; k < glen; ++k) {
        h[k] = sigm(est_logit(A.est, k + 1 < 15 ? k + 1 : 15, n, am, m));
        s *= h[k];
        Sg[k] = s;
    }
    s = 1.0;
    for (int k = 0; k < K; ++k) {
        const double cv = (double)A.model_conf[(int64_t)r * K + k];
        s *= A.conf_is_logit ? sigm(cv) : cv;
        Sd[k] = s;
    }
    const int32_t* d = A.model_tokens + (int64_t)r * K;
    const int32_t* g = A.ngram_draft + (int64_t)r * A.ngram_ld;
    bool prefix = glen > K;
    for (int i = 0; prefix && i < K; ++i) prefix = (g[i] == d[i]);
    int use = SPEC_SRC_MODEL;
    switch (A.policy) {
    case SPEC_POLICY_PROPOSED:
        if (prefix) use = SPEC_SRC_MERGED;
        else if (glen >= 1) use = (chain_value(Sg, glen, (double)A.lambda) >= chain_value(Sd, K, (double)A.lambda)) ? SPEC_SRC_NGRAM : SPEC_SRC_MODEL;
        break;
    case SPEC_POLICY_NGRAM_FIRST: use = glen >= 1 ? SPEC_SRC_NGRAM : SPEC_SRC_MODEL; break;
    case SPEC_POLICY_EXTENSION: use = prefix ? SPEC_SRC_EXTENDED : SPEC_SRC_MODEL; break;
    case SPEC_POLICY_NGRAM_ONLY: use = SPEC_SRC_NGRAM; break;
    default: use = SPEC_SRC_MODEL;
    }
    const bool mpm = !A.model_point_mass || A.model_point_mass[r];
    const uint8_t mfl = mpm ? SPEC_SLOT_POINT_MASS : 0;
    const uint8_t gfl = SPEC_SLOT_POINT_MASS | SPEC_SLOT_FROM_NGRAM;
    const int len = (use == SPEC_SRC_MODEL) ? K : glen;
    double prev = 1.0;
    for (int k = 0; k < ld; ++k) {
        int32_t tk = -1;
        uint8_t fl = 0;
        double S = 0.0;
        if (k < len) {
            if (use == SPEC_SRC_MODEL) { tk = d[k]; fl = mfl; S = Sd[k]; }
            else if (use == SPEC_SRC_NGRAM) { tk = g[k]; fl = gfl; S = Sg[k]; }
            else if (use == SPEC_SRC_MERGED) { tk = g[k]; fl = gfl; S = (k < K) ? (Sg[k] > Sd[k] ? Sg[k] : Sd[k]) : prev * h[k]; }
            else { tk = g[k]; if (k < K) { fl = mfl; S = Sd[k]; } else { fl = gfl; S = prev * h[k]; } }
            prev = S;
        }
        const int64_t o = (int64_t)r * ld + k;
        A.chain_tokens[o] = tk;
        A.slot_flags[o] = fl;
        A.survival[o] = (float)S;
        uint64_t key = 0;
        if (k < len) {
            const float sf = (float)S;
            key = ((uint64_t)__float_as_uint(sf) << 32) | ((uint64_t)(31 - k) << 27) | (uint64_t)(0x7FFFFFF - r);
        }
        P.keys[o] = key;
    }
    A.chain_len[r] = len;
    A.chain_src[r] = use;
    A.out_flags[r] = flags;
}

constexpr int kTopkBlock = 1024;

__device__ int64_t block_exclusive_i64(int64_t v, int64_t* total)
{
    __shared__ int64_t sh[kTopkBlock / kWave];
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
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
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) {
        if (w < wid) before += sh[w];
        tot += sh[w];
    }
    *total = tot;
    return before + inc - v;
}

__global__ __launch_bounds__(kTopkBlock) void k_topk(SelectParams P)
{
    const spec_chain_alloc& A = P.a;
    const int64_t N = (int64_t)A.bs * A.ld;
    __shared__ uint32_t hist[256];
    __shared__ uint64_t sh_prefix, sh_mask;
    __shared__ int64_t sh_rem, sh_valid;
    if (threadIdx.x == 0) { sh_prefix = 0; sh_mask = 0; sh_valid = 0; }
    __syncthreads();
    // number of real slots
    {
        int64_t c = 0;
        for (int64_t i = threadIdx.x; i < N; i += kTopkBlock) c += P.keys[i] != 0;
        atomicAdd((unsigned long long*)&sh_valid, (unsigned long long)c);
    }
    __syncthreads();
    const int64_t take = (A.budget < sh_valid) ? A.budget : sh_valid;
    uint64_t theta = ~0ull;  // nothing selected
    if (take > 0) {
        if (threadIdx.x == 0) sh_rem = take;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = threadIdx.x; i < 256; i += kTopkBlock) hist[i] = 0;
            __syncthreads();
            const uint64_t pre = sh_prefix, msk = sh_mask;
            for (int64_t i = threadIdx.x; i < N; i += kTopkBlock) {
                const uint64_t k = P.keys[i];
                if (k != 0 && (k & msk) == pre) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                int64_t rem = sh_rem, cum = 0;
                int dsel = 0;
                for (int dg = 255; dg >= 0; --dg) {
                    if (cum + hist[dg] >= rem) { dsel = dg; break; }
                    cum += hist[dg];
                }
                sh_rem = rem - cum;
                sh_prefix = pre | ((uint64_t)dsel << shift);
                sh_mask = msk | (255ull << shift);
            }
            __syncthreads();
        }
        theta = sh_prefix;
    }
    // per-request verified prefix, then CSR row bases over (alloc + 1)
    const int bs = A.bs;
    const int per = (bs + kTopkBlock - 1) / kTopkBlock;
    const int r0 = threadIdx.x * per;
    int64_t local = 0;
    for (int r = r0; r < r0 + per && r < bs; ++r) {
        int cnt = 0;
        for (int k = 0; k < A.ld; ++k) {
            const uint64_t key = P.keys[(int64_t)r * A.ld + k];
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
    if (lane == 0) {
        fsel[0] = 1;
        // depth-first layout, children in index order
        int st_n[SPEC_MAX_ROWS], st_p[SPEC_MAX_ROWS];
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

__global__ __launch_bounds__(kTopkBlock) void k_rows_scan(const int32_t* n_rows, int bs, int64_t* row_base, int32_t* total_rows)
{
    const int per = (bs + kTopkBlock - 1) / kTopkBlock;
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
    if (a->mode == SPEC_ALLOC_CHAIN) return align256((size_t)a->chain.bs * a->chain.ld * sizeof(uint64_t));
    return 0;
}

int spec_alloc_launch(const spec_alloc_args* a, hipStream_t st)
{
    if (a->mode == SPEC_ALLOC_CHAIN) {
        SelectParams P;
        P.a = a->chain;
        P.keys = (uint64_t*)a->workspace;
        hipLaunchKernelGGL(k_select, dim3((a->chain.bs + 63) / 64), dim3(64), 0, st, P);
        hipLaunchKernelGGL(k_topk, dim3(1), dim3(kTopkBlock), 0, st, P);
    } else {
        TreeBuildParams P;
        P.a = a->tree;
        hipLaunchKernelGGL(k_tree, dim3(a->tree.bs), dim3(kWave), 0, st, P);
        hipLaunchKernelGGL(k_rows_scan, dim3(1), dim3(kTopkBlock), 0, st, a->tree.n_rows, a->tree.bs, a->tree.row_base,
                           a->tree.total_rows);
    }
    return spec_record_hip_error(hipGetLastError());
}
