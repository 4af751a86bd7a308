// Budget sizing and slot price: host arithmetic over the survivals of the
// batch's chosen chains (Hybrid Spark, Section 2 "Adaptive verification" and
// "Asynchronous scheduling", Section 4.3 Eq. (2), Appendix F with Eq. (4)).
// The survivals are ordered by a three-pass radix sort of their bit patterns
// (non-negative floats order like their bits; negatives, NaN and padding
// count as 0), after which the goodput of every budget is one pass of prefix
// sums.  It runs on the host between steps, so it must cost far less than a
// step: a few microseconds for a batch's few thousand survivals.
#include <cmath>
#include <cstring>
#include <vector>

#include "spec.h"

namespace {

// Keys in descending order of value: the complement of the bits ascending.
void sort_desc(const float* in, int64_t n, std::vector<uint32_t>& a, std::vector<uint32_t>& b)
{
    a.resize(n);
    b.resize(n);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t x;
        std::memcpy(&x, &in[i], 4);
        const bool pos = in[i] > 0.0f;          // false for NaN too
        a[i] = ~(pos ? x : 0u);
    }
    constexpr int kBits = 11;
    constexpr uint32_t kMask = (1u << kBits) - 1;
    uint32_t cnt[1u << kBits];
    for (int shift = 0; shift < 32; shift += kBits) {
        std::memset(cnt, 0, sizeof(cnt));
        for (int64_t i = 0; i < n; ++i) ++cnt[(a[i] >> shift) & kMask];
        uint32_t sum = 0;
        for (uint32_t d = 0; d <= kMask; ++d) {
            const uint32_t c = cnt[d];
            cnt[d] = sum;
            sum += c;
        }
        for (int64_t i = 0; i < n; ++i) b[cnt[(a[i] >> shift) & kMask]++] = a[i];
        a.swap(b);
    }
}

// C(b), or a negative value when the step cannot run with b draft slots.
double step_cost(const spec_cost_model& cm, int64_t b)
{
    double c = cm.c0 + cm.p * (double)b;
    if (cm.graph_limit > 0 && (int64_t)cm.n_tokens + b > cm.graph_limit) {
        const int64_t k = (int64_t)cm.n_tokens + b - cm.graph_limit - 1;
        if (k >= cm.n_eager) return -1.0;
        c = std::max(c, cm.eager[k]);
    }
    return c;
}

}  // namespace

extern "C" int spec_size_budget(const float* survival, int64_t n, int32_t n_requests, const spec_cost_model* cost,
                                int32_t b_max, int32_t* b_star, double* lambda, double* goodput, double* curve)
{
    if (!cost || !b_star || !lambda || n < 0 || (n > 0 && !survival) || n_requests < 0) return SPEC_EINVAL;
    if (!(cost->c0 > 0.0) || !(cost->p >= 0.0) || !std::isfinite(cost->c0) || !std::isfinite(cost->p))
        return SPEC_EINVAL;
    if (cost->graph_limit < 0 || cost->n_tokens < 0 || cost->n_eager < 0 || (cost->n_eager > 0 && !cost->eager))
        return SPEC_EINVAL;
    const int64_t top = (b_max <= 0 || b_max > n) ? n : b_max;
    thread_local std::vector<uint32_t> ka, kb;   // host scratch, reused by the calling thread
    sort_desc(survival, n, ka, kb);
    double A = (double)n_requests;
    int64_t best = -1;
    double abest = 0.0, cbest = 1.0;
    for (int64_t b = 0; b <= top; ++b) {
        if (b > 0) {
            const uint32_t bits = ~ka[b - 1];
            float v;
            std::memcpy(&v, &bits, 4);
            A += (double)v;
        }
        const double c = step_cost(*cost, b);
        if (curve) curve[b] = c > 0.0 ? A / c : -1.0;
        // G(b) > G(best), compared without dividing; the quotients decide
        // only when the products are too close to tell them apart
        if (c > 0.0) {
            bool better = best < 0;
            if (!better) {
                const double l = A * cbest, r = abest * c;
                better = l > r * (1.0 + 1e-12) || (l >= r * (1.0 - 1e-12) && A / c > abest / cbest);
            }
            if (better) {
                best = b;
                abest = A;
                cbest = c;
            }
        }
    }
    const double g = best < 0 ? 0.0 : abest / cbest;
    *b_star = (int32_t)(best < 0 ? 0 : best);
    *lambda = g * cost->p;
    if (goodput) *goodput = g;
    return SPEC_OK;
}
