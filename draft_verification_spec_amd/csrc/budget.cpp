// Budget sizing and slot price: host arithmetic over the survivals of the
// batch's chosen chains (Hybrid Spark, Section 2 "Adaptive verification" and
// "Asynchronous scheduling", Section 4.3 Eq. (2), Appendix F with Eq. (4)).
// Only the b_max largest survivals matter, so they alone are ordered (a
// partial sort); the goodput of every budget is then one pass of prefix sums.
#include <algorithm>
#include <cmath>
#include <functional>
#include <vector>

#include "spec.h"

namespace {

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
    std::vector<float> s(survival, survival + n);
    for (float& x : s) x = x > 0.0f ? x : 0.0f;   // NaN and padding add nothing
    std::partial_sort(s.begin(), s.begin() + top, s.end(), std::greater<float>());
    double A = (double)n_requests;
    int64_t best = -1;
    double gbest = -1.0;
    for (int64_t b = 0; b <= top; ++b) {
        if (b > 0) A += (double)s[b - 1];
        const double c = step_cost(*cost, b);
        const double g = c > 0.0 ? A / c : -1.0;
        if (curve) curve[b] = g;
        if (g >= 0.0 && (best < 0 || g > gbest)) {
            best = b;
            gbest = g;
        }
    }
    *b_star = (int32_t)(best < 0 ? 0 : best);
    *lambda = best < 0 ? 0.0 : gbest * cost->p;
    if (goodput) *goodput = best < 0 ? 0.0 : gbest;
    return SPEC_OK;
}
