// The n-gram scan of one query by one workgroup of NT threads (Hybrid Spark,
// Section 4.1 "One step" and Section 4.2 match features; Algorithm 1,
// NGRAMSCAN), shared by the drafter kernel and by the chain verifier, which
// drafts each request's next n-gram chain right after its commit.
//
//   * each thread tests end positions j = t, t + NT, ...: it loads the token at
//     j for a batch of 16 positions (independent coalesced loads, one memory
//     round trip per batch) and the batch (16 NT tokens) is staged in LDS, so
//     that every later comparison reads LDS;
//   * the query's trailing copy_cap tokens are staged in LDS as well, from the
//     window when the whole text fits in it;
//   * for the rare hits a thread compares up to 4 tokens backwards itself;
//     positions still matching after 4 go to a candidate list that whole waves
//     extend 64 tokens per step with a ballot (compared up to
//     min(j + 1, copy_cap));
//   * a match of length l >= n_min becomes the key (l << 32 | j), so "longest,
//     then latest" is the largest key; the workgroup keeps the top two;
//   * thread 0 derives (n, a, m, j) and the first lanes copy the draft, from
//     the window when it holds the continuation;
//   * with the follower fallback (AdaSpark, Section 3.3, "N-gram candidates"),
//     each further token after the copy is the most frequent follower of the
//     last F tokens: every thread tests its positions against the context and
//     counts the followers in an LDS hash table (token -> count, latest
//     position), and the largest (count, latest) wins.
#pragma once

#include "common.hpp"

namespace spec {

constexpr int kBatch = 16;       // positions per thread per batch (at most 32: a bit mask of hits)
constexpr int kPre = 4;          // tokens each thread compares before handing a match to its wave
constexpr int kMaxCand = 2048;   // candidate list in LDS; overflow is extended by the thread itself

struct Text {
    const int32_t* a;  // context row
    int64_t na;
    const int32_t* b;  // extra row (may be null)
    int64_t n;         // total length
};

// Token p of the text: the address is selected first, so a batch of these is
// a batch of independent loads rather than branches around them.  The load
// goes through a global-memory pointer: the integer arithmetic would
// otherwise leave a generic one, i.e. a flat load that waits for every
// outstanding access (LDS ones included).
__device__ __forceinline__ int32_t tok(const Text& x, int64_t p)
{
    const uintptr_t pa = (uintptr_t)(x.a + p);
    const uintptr_t pb = (uintptr_t)x.b + (uintptr_t)((p - x.na) * (int64_t)sizeof(int32_t));
    return *(const __attribute__((address_space(1))) int32_t*)(p < x.na ? pa : pb);
}

template <int NT, int NCAND = kMaxCand>
struct NgramShared {
    int32_t suf[SPEC_MAX_CAP];
    Top2 sh[NT / kWave];
    int32_t cand[NCAND];
    int32_t n_cand;
};

struct NgramOut {
    int32_t n_min, n_max, max_draft, cap;
    int32_t* draft;      // [max_draft]
    int32_t* draft_len;  // [1]
    int32_t* feat;       // [4]
    int32_t follow_ctx;  // F > 0: the follower fallback (needs a FollowShared)
    int32_t* follow;     // [max_draft] follower counts, or null
};

// LDS of the follower fallback beyond the scan's own (whose suffix and
// candidate lists hold the hash table's counts and keys).
constexpr int kFollowers = SPEC_MAX_FOLLOWERS;
static_assert(kMaxCand * sizeof(int32_t) >= kFollowers * sizeof(uint64_t), "hash keys fit the full candidate list");
static_assert(SPEC_MAX_CAP >= kFollowers, "hash counts fit the suffix");
struct FollowShared {
    int32_t last[kFollowers];       // latest position of each follower
    int32_t dft[SPEC_MAX_DRAFT];    // the draft so far
    int32_t fol[SPEC_MAX_DRAFT];    // follower counts
    uint64_t best[16];              // per wave: (count << 32 | latest position)
    int32_t len, over;
};

// Scans text x with the whole workgroup (every thread calls it): batches of
// NB positions per thread (NT * NB positions), of which the first NWIN per
// thread are staged in win (NT * NWIN tokens of LDS); the rest of a batch is
// tested from registers and read from memory where needed.  With `pre`, v
// already holds the first batch (positions t + u * NT, any value past the
// text).  NCAND bounds the LDS list of candidates extended by whole waves.
template <int NT, int NB = kBatch, int NWIN = NB, int NCAND = kMaxCand>
__device__ __forceinline__ void ngram_scan(const Text& x, int32_t* win, NgramShared<NT, NCAND>& S, const NgramOut& O,
                           int32_t (&v)[NB], bool pre, FollowShared* FS = nullptr)
{
    static_assert(NT / kWave <= 16, "per-wave slots of FollowShared");
    static_assert(NWIN >= 1 && NWIN <= NB, "the window is a prefix of the batch");
    constexpr int64_t kWin = (int64_t)NT * NWIN;    // tokens staged in LDS
    constexpr int64_t kSpan = (int64_t)NT * NB;     // positions per batch
    const int t = threadIdx.x;
    const int lane = t % kWave, wid = t / kWave;
    const int64_t jend = x.n - 1;                 // end positions j < n - 1
    const int64_t ns = x.n < O.cap ? x.n : O.cap;
    // batch loads: kBatch independent loads per thread; past the text they
    // read its last position (in bounds) and are masked off later, so a
    // window holds every position of the text it covers
    auto load_batch = [&](int64_t base) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int64_t j = base + t + (int64_t)u * NT;
            v[u] = tok(x, j < x.n ? j : x.n - 1);
        }
    };
    if (!pre && jend > 0) load_batch(0);   // in flight while the suffix is staged
    const bool suf_in_win = x.n <= kWin;
    if (!suf_in_win)
        for (int64_t i = t; i < ns; i += NT) S.suf[i] = tok(x, x.n - 1 - i);
    if (t == 0) S.n_cand = 0;
    // token at position p < n: from the staged window when it holds p
    int64_t wbase = 0;
    auto at = [&](int64_t p) -> int32_t { return (p >= wbase && p < wbase + kWin) ? win[p - wbase] : tok(x, p); };
    Top2 best{0, 0};
    if (jend > 0) {
        // phase 1: first kPre tokens per position, thread-private
        for (int64_t base = 0; base < jend; base += kSpan) {
            if (base > 0) {
                __syncthreads();   // the previous window is no longer read
                load_batch(base);
            }
#pragma unroll
            for (int u = 0; u < NWIN; ++u) win[t + u * NT] = v[u];
            wbase = base;
            __syncthreads();
            if (base == 0 && suf_in_win) {
                for (int64_t i = t; i < ns; i += NT) S.suf[i] = win[x.n - 1 - i];
                __syncthreads();
            }
            static_assert(kPre == 4, "the first check reads three tokens back");
            const int32_t s0 = S.suf[0], s1 = S.suf[1], s2 = S.suf[2], s3 = S.suf[3];
            uint32_t hits = 0;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int64_t j = base + t + (int64_t)u * NT;
                hits |= (uint32_t)(j < jend && v[u] == s0) << u;
            }
            // one text in one window (the usual case): its tokens straight from LDS
            const bool whole = suf_in_win;
            // A hit whose previous token differs from s1 has l = 1, which
            // matters only when n_min is 1.  With the text in the window, a
            // wave that has hits reads every previous token at once (one
            // independent LDS read per batch slot) and drops those hits, so a
            // frequent last token does not cost a loop round per hit.
            if (whole && O.n_min >= 2 && __ballot(hits != 0u) != 0) {
                uint32_t keep = 0;
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const int64_t j = t + (int64_t)u * NT;
                    keep |= (uint32_t)(win[j >= 1 ? j - 1 : 0] == s1) << u;
                }
                hits &= keep;
            }
            while (hits) {
                const int u = __builtin_ctz(hits);
                hits &= hits - 1;
                const int64_t j = base + t + (int64_t)u * NT;
                const int64_t lim = (j + 1 < O.cap) ? j + 1 : O.cap;
                // the three tokens before j read together (positions below 0
                // read position 0; lim keeps them out of the count), then the
                // run of matches they start: l as the token-by-token check
                // up to kPre would find it
                int32_t b1, b2, b3;
                if (whole) {
                    b1 = win[j >= 1 ? j - 1 : 0];
                    b2 = win[j >= 2 ? j - 2 : 0];
                    b3 = win[j >= 3 ? j - 3 : 0];
                } else {
                    b1 = at(j >= 1 ? j - 1 : 0);
                    b2 = at(j >= 2 ? j - 2 : 0);
                    b3 = at(j >= 3 ? j - 3 : 0);
                }
                int64_t l = 1;
                if (l < lim && b1 == s1) {
                    l = 2;
                    if (l < lim && b2 == s2) {
                        l = 3;
                        if (l < lim && b3 == s3) l = 4;
                    }
                }
                if (l == kPre && l < lim) {
                    const int c = atomicAdd(&S.n_cand, 1);
                    if (c < NCAND) {
                        S.cand[c] = (int32_t)j;
                        continue;
                    }
                    while (l < lim && at(j - l) == S.suf[l]) ++l;   // list full: extend here
                }
                if (l >= O.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)j);
            }
        }
    }
    __syncthreads();
    // phase 2: the listed candidates, four per wave (16 lanes each) for their
    // 16 tokens past kPre (most stop there); each one still matching then
    // takes the whole wave, 64 tokens per step
    const int nc = S.n_cand < NCAND ? S.n_cand : NCAND;
    constexpr int kSeg = 16, kSegs = kWave / kSeg;
    const int sub = lane / kSeg, sl = lane % kSeg;
    for (int c0 = wid * kSegs; c0 < nc; c0 += (NT / kWave) * kSegs) {
        const int c = c0 + sub;
        const bool has = c < nc;
        const int32_t j = has ? S.cand[c] : 0;
        const int32_t lim = has ? ((j + 1 < O.cap) ? j + 1 : O.cap) : 0;
        const int64_t i0 = kPre + sl;
        const bool eq0 = i0 < lim && at(j - i0) == S.suf[i0];
        const uint32_t seg = (uint32_t)(__ballot(eq0) >> (sub * kSeg)) & 0xFFFFu;
        const bool longer = has && seg == 0xFFFFu;
        if (has && sl == 0 && !longer) {
            int64_t l = kPre + __builtin_ctz(~seg);
            if (l > lim) l = lim;
            if (l >= O.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)j);
        }
        for (uint64_t lm = __ballot(longer && sl == 0); lm; lm &= lm - 1) {
            const int g = (int)__builtin_ctzll(lm);
            const int32_t jj = __builtin_amdgcn_readlane(j, g), ll = __builtin_amdgcn_readlane(lim, g);
            int64_t l = kPre + kSeg;
            for (;;) {
                const int64_t i = l + lane;
                const bool eq = i < ll && at(jj - i) == S.suf[i];
                const uint64_t miss = ~__ballot(eq);
                if (miss == 0) {
                    l += kWave;
                    continue;
                }
                l += (int64_t)__builtin_ctzll(miss);
                break;
            }
            if (l > ll) l = ll;
            if (lane == 0 && l >= O.n_min) best = top2_insert(best, ((uint64_t)l << 32) | (uint64_t)jj);
        }
    }
    best = wave_top2(best);
    if (lane == 0) S.sh[wid] = best;
    __syncthreads();
    const bool follow = O.follow_ctx > 0 && FS != nullptr;
    if (wid == 0) {
        Top2 tb = lane < NT / kWave ? S.sh[lane] : Top2{0, 0};
        tb = wave_top2(tb);
        int32_t* d = O.draft;
        if (tb.a == 0) {
            for (int k = lane; k < O.max_draft; k += kWave) {
                d[k] = -1;
                if (follow) FS->dft[k] = -1;
            }
            if (lane == 0) {
                *O.draft_len = 0;
                if (follow) FS->len = 0;
                O.feat[0] = 0;
                O.feat[1] = 0;
                O.feat[2] = 0;
                O.feat[3] = -1;
            }
        } else {
            const int64_t l = (int64_t)(tb.a >> 32);
            const int64_t j = (int64_t)(tb.a & 0xFFFFFFFFu);
            const int64_t avail = x.n - 1 - j;
            const int64_t len = avail < O.max_draft ? avail : O.max_draft;
            for (int k = lane; k < O.max_draft; k += kWave) {
                const int32_t tk = (k < len) ? at(j + 1 + k) : -1;
                d[k] = tk;
                if (follow) FS->dft[k] = tk;
            }
            if (lane == 0) {
                int a = 1;
                if (tb.b != 0) {
                    const int64_t jr = (int64_t)(tb.b & 0xFFFFFFFFu);
                    a = at(jr + 1) == at(j + 1);
                }
                *O.draft_len = (int32_t)len;
                if (follow) FS->len = (int32_t)len;
                O.feat[0] = (int32_t)(l < O.n_max ? l : O.n_max);
                O.feat[1] = a;
                O.feat[2] = (l >= O.n_max) ? (int32_t)l : 0;
                O.feat[3] = (int32_t)j;
            }
        }
    }
    if constexpr (NCAND * sizeof(int32_t) < kFollowers * sizeof(uint64_t)) {
        return;   // no room for the follower hash: instances with NCAND this small never take the fallback
    } else {
    if (!follow) return;
    // follower fallback: one token per round while the draft is short
    __syncthreads();
    const int F = O.follow_ctx;
    uint64_t* hkey = (uint64_t*)S.cand;   // (1 << 32 | token), 0 = empty
    int32_t* hcnt = S.suf;
    const int len0 = FS->len;
    int len = len0;
    // no copy and F >= n_min: every occurrence of the last F tokens would
    // have been a match, so there is no follower either
    const bool none = len0 == 0 && F >= O.n_min;
    while (!none && len < O.max_draft && x.n + len >= F) {
        for (int i = t; i < kFollowers; i += NT) {
            hkey[i] = 0;
            hcnt[i] = 0;
            FS->last[i] = -1;
        }
        if (t == 0) FS->over = 0;
        __syncthreads();
        int32_t c[SPEC_MAX_FOLLOW_CTX];
#pragma unroll
        for (int i = 0; i < SPEC_MAX_FOLLOW_CTX; ++i) {
            const int64_t q = x.n + len - F + i;   // position in text ++ draft
            c[i] = i < F ? (q < x.n ? at(q) : FS->dft[q - x.n]) : 0;
        }
        for (int64_t p = F - 1 + t; p + 1 < x.n; p += NT) {
            bool m = true;
            for (int i = 0; i < F && m; ++i) m = at(p - (F - 1) + i) == c[i];
            if (!m) continue;
            const int32_t f = at(p + 1);
            const uint64_t key = (1ull << 32) | (uint32_t)f;
            uint32_t h = ((uint32_t)f * 2654435761u) >> 22;   // 10 bits: kFollowers slots
            int probe = 0;
            for (; probe < kFollowers; ++probe) {
                const uint64_t old = atomicCAS((unsigned long long*)&hkey[h], 0ull, (unsigned long long)key);
                if (old == 0 || old == key) {
                    atomicAdd(&hcnt[h], 1);
                    atomicMax(&FS->last[h], (int32_t)p);
                    break;
                }
                h = (h + 1) & (kFollowers - 1);
            }
            if (probe == kFollowers) FS->over = 1;   // more distinct followers than the table holds
        }
        __syncthreads();
        uint64_t b = 0;
        for (int i = t; i < kFollowers; i += NT) {
            const uint64_t e = hcnt[i] > 0 ? ((uint64_t)(uint32_t)hcnt[i] << 32) | (uint32_t)FS->last[i] : 0ull;
            b = e > b ? e : b;
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)b, o, kWave), hi = __shfl_xor((uint32_t)(b >> 32), o, kWave);
            const uint64_t y = ((uint64_t)hi << 32) | lo;
            b = y > b ? y : b;
        }
        if (lane == 0) FS->best[wid] = b;
        __syncthreads();
        if (t == 0) {
            uint64_t bb = 0;
            for (int w = 0; w < NT / kWave; ++w) bb = FS->best[w] > bb ? FS->best[w] : bb;
            if (bb == 0 || FS->over) {
                FS->over = 1;   // the draft ends here
            } else {
                const int64_t plast = (int64_t)(uint32_t)bb;
                FS->dft[len] = at(plast + 1);
                FS->fol[len] = (int32_t)(bb >> 32);
            }
        }
        __syncthreads();
        if (FS->over) break;
        ++len;
    }
    // the fallback's tokens and every count
    for (int k = t; k < O.max_draft; k += NT) {
        if (k >= len0 && k < len) O.draft[k] = FS->dft[k];
        if (O.follow) O.follow[k] = (k >= len0 && k < len) ? FS->fol[k] : 0;
    }
    if (t == 0) *O.draft_len = len;
    }
}

}  // namespace spec
