// Host-only exercise of the library's host code and of the C oracle, built by
// tests/test_sanitize_cpu.py with AddressSanitizer and UndefinedBehavior-
// Sanitizer (any finding aborts).  It runs the budget sizing over random and
// edge-case survivals and cost tables, every argument validation with good
// and bad arguments, and the oracle's functions on small inputs, checking a
// few results on the way.  No GPU, no HIP.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "spec.h"
#include "validate.hpp"

extern "C" {
// the oracle's C entry points (oracle/spec_oracle.c)
void oracle_ngram_draft(int nq, const int32_t* ctx, int64_t ctx_stride, const int32_t* ctx_len,
                        const int32_t* query_req, const int32_t* extra, int64_t extra_stride,
                        const int32_t* extra_len, int n_min, int n_max, int max_draft, int cap, int follow_ctx,
                        int32_t* draft, int32_t* draft_len, int32_t* feat, int32_t* follow);
int oracle_select(int K, const int32_t* d, const double* c, int dlen, const int32_t* g, const double* h, int glen,
                  double lambda, int policy, int model_point_mass, int ld, int32_t* out_tok, uint8_t* out_flag,
                  double* out_S, int32_t* out_src, int* near);
void oracle_allocate(int bs, int ld, const int32_t* len, const double* S, int budget, int32_t* alloc,
                     int64_t* row_base, int32_t* total, uint32_t* flags);
void oracle_verify_chain(int bs, int V, double T, const void* logits, int dtype, int64_t row_stride,
                         const int64_t* row_base, const void* dlogits, int ddtype, int64_t drow_stride,
                         const int64_t* drow_base, const int32_t* tokens, const uint8_t* slot_flags, int ld,
                         const int32_t* n_slots, const float* u_acc, const float* u_smp, int32_t* out_tokens,
                         int32_t* out_num, int32_t* out_accepted, double* out_p, double* out_q,
                         uint32_t* out_flags, int32_t* out_win_lo, int32_t* out_win_hi);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
int oracle_tree_forest(int n, int c_max, const int32_t* token, const int32_t* parent, const float* q, int rows_cap,
                       int32_t* node_token, int32_t* parent_row, double* Q_out, int32_t* n_rows, double* S_curve,
                       double* f_Q, uint32_t* flag);
}

static unsigned g_seed = 12345u;
static unsigned rnd() { g_seed = g_seed * 1664525u + 1013904223u; return g_seed >> 8; }
static double urand() { return (rnd() & 0xFFFFFF) / 16777216.0; }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); return 1; } } while (0)

static int budget_sizing()
{
    for (int trial = 0; trial < 300; ++trial) {
        const int n = 1 + (int)(rnd() % 400);
        std::vector<float> S(n);
        for (int i = 0; i < n; ++i) {
            const unsigned k = rnd() % 10;
            S[i] = k == 0 ? -0.5f : (k == 1 ? NAN : (k == 2 ? 0.0f : (float)urand()));
        }
        std::vector<double> eager(1 + rnd() % 8);
        for (size_t i = 0; i < eager.size(); ++i) eager[i] = 100.0 + 10.0 * i + urand();
        spec_cost_model cm;
        cm.c0 = 50.0 + urand() * 50.0;
        cm.p = urand();
        cm.graph_limit = (trial % 3 == 0) ? 0 : (int32_t)(rnd() % 300);
        cm.n_tokens = (int32_t)(rnd() % 64);
        cm.eager = eager.data();
        cm.n_eager = (int32_t)eager.size();
        const int32_t b_max = (trial % 4 == 0) ? 0 : (int32_t)(rnd() % (n + 5));
        const int top = (b_max <= 0 || b_max > n) ? n : b_max;
        std::vector<double> curve(top + 1);
        int32_t b = -1;
        double lam = -1.0, gb = -1.0;
        const int rc = spec_size_budget(S.data(), n, 1 + (int)(rnd() % 64), &cm, b_max, &b, &lam, &gb, curve.data());
        CHECK(rc == SPEC_OK);
        CHECK(b >= 0 && b <= top);
        CHECK(curve[b] == gb || (gb == 0.0 && b == 0 && curve[0] < 0));   // no budget can run: b* = 0, G = 0
        for (int i = 0; i <= top; ++i) CHECK(curve[i] <= gb || curve[i] < 0);
    }
    // bad arguments
    spec_cost_model cm = {1.0, 0.1, 0, 0, nullptr, 0};
    int32_t b;
    double lam;
    float s1 = 0.5f;
    CHECK(spec_size_budget(nullptr, 1, 1, &cm, 0, &b, &lam, nullptr, nullptr) == SPEC_EINVAL);
    CHECK(spec_size_budget(&s1, 1, 1, nullptr, 0, &b, &lam, nullptr, nullptr) == SPEC_EINVAL);
    cm.c0 = -1.0;
    CHECK(spec_size_budget(&s1, 1, 1, &cm, 0, &b, &lam, nullptr, nullptr) == SPEC_EINVAL);
    return 0;
}

static int validation()
{
    using namespace spec_validate;
    int32_t dummy[64] = {0};
    spec_ngram_args ng;
    memset(&ng, 0, sizeof ng);
    CHECK(check_ngram(nullptr) == SPEC_EINVAL);
    CHECK(check_ngram(&ng) == SPEC_EINVAL);
    ng.bs = 2; ng.nq = 2; ng.ctx = dummy; ng.ctx_stride = 8; ng.ctx_len = dummy;
    ng.n_min = 3; ng.n_max = 15; ng.max_draft = 15; ng.copy_cap = 256;
    ng.draft = dummy; ng.draft_len = dummy; ng.feat = dummy;
    CHECK(check_ngram(&ng) == SPEC_OK);
    ng.max_draft = SPEC_MAX_DRAFT + 1;
    CHECK(check_ngram(&ng) == SPEC_EINVAL);
    ng.max_draft = 15; ng.copy_cap = 2;
    CHECK(check_ngram(&ng) == SPEC_EINVAL);

    spec_verify_args v;
    memset(&v, 0, sizeof v);
    CHECK(check_verify(&v) == SPEC_EINVAL);
    v.bs = 4; v.vocab = 100; v.temperature = 1.0f; v.logits = dummy; v.dtype = SPEC_BF16; v.row_stride = 100;
    v.row_base = (const int64_t*)dummy; v.n_logit_rows = 10; v.tokens = dummy; v.n_slots = dummy; v.ld = 7;
    v.u_accept = (const float*)dummy; v.u_sample = (const float*)dummy;
    v.out_tokens = dummy; v.out_num = dummy; v.out_accepted = dummy; v.out_flags = (uint32_t*)dummy;
    CHECK(check_verify(&v) == SPEC_OK);
    v.dtype = 7;
    CHECK(check_verify(&v) == SPEC_EINVAL);
    v.dtype = SPEC_F32; v.temperature = -1.0f;
    CHECK(check_verify(&v) == SPEC_EINVAL);
    v.temperature = 0.0f; v.u_accept = nullptr; v.u_sample = nullptr;
    CHECK(check_verify(&v) == SPEC_OK);   // greedy needs no uniforms
    v.ld = SPEC_MAX_DRAFT + 1;
    CHECK(check_verify(&v) == SPEC_EINVAL);

    spec_tree_verify_args tv;
    memset(&tv, 0, sizeof tv);
    CHECK(check_tree_verify(&tv) == SPEC_EINVAL);
    spec_alloc_args al;
    memset(&al, 0, sizeof al);
    al.mode = 9;
    CHECK(check_alloc(&al) == SPEC_EINVAL);
    al.mode = SPEC_ALLOC_CHAIN;
    CHECK(check_alloc(&al) == SPEC_EINVAL);
    al.mode = SPEC_ALLOC_TREE;   // a caller-built forest
    al.tree.bs = 3; al.tree.c_max = 40; al.tree.rows_cap = 16;
    al.tree.node_token = dummy; al.tree.parent_row = dummy; al.tree.Q = (float*)dummy; al.tree.n_rows = dummy;
    al.tree.row_base = (int64_t*)dummy; al.tree.total_rows = dummy; al.tree.forest_count = dummy;
    al.tree.out_flags = (uint32_t*)dummy;
    al.tree.forest_token = dummy;
    CHECK(check_alloc(&al) == SPEC_EINVAL);
    al.tree.forest_parent = dummy; al.tree.forest_q = (const float*)dummy; al.tree.forest_n = dummy;
    CHECK(check_alloc(&al) == SPEC_OK);
    al.tree.c_max = SPEC_MAX_FOREST + 1;
    CHECK(check_alloc(&al) == SPEC_EINVAL);
    al.tree.c_max = 40; al.tree.rows_cap = SPEC_MAX_ROWS + 1;
    CHECK(check_alloc(&al) == SPEC_EINVAL);
    CHECK(check_workspace(nullptr, 0, 0) == SPEC_OK);
    CHECK(check_workspace(nullptr, 0, 16) == SPEC_EWORKSPACE);
    CHECK(check_workspace((void*)(uintptr_t)0x1000, 8, 16) == SPEC_EWORKSPACE);
    CHECK(check_workspace((void*)(uintptr_t)0x1008, 64, 16) == SPEC_EWORKSPACE);
    return 0;
}

static int oracle_functions()
{
    // n-gram draft on random texts over a small alphabet
    for (int trial = 0; trial < 200; ++trial) {
        const int T = 1 + (int)(rnd() % 300), nq = 3;
        std::vector<int32_t> ctx(nq * 300), len(nq), draft(nq * 15), dl(nq), feat(nq * 4), fol(nq * 15);
        for (auto& x : ctx) x = (int32_t)(rnd() % 3);
        for (int q = 0; q < nq; ++q) len[q] = T - q < 0 ? 0 : T - q;
        oracle_ngram_draft(nq, ctx.data(), 300, len.data(), nullptr, nullptr, 0, nullptr, 2, 15, 15, 256,
                           trial % 2 ? 3 : 0, draft.data(), dl.data(), feat.data(), fol.data());
        for (int q = 0; q < nq; ++q) CHECK(dl[q] >= 0 && dl[q] <= 15);
    }
    // selection and allocation
    for (int trial = 0; trial < 200; ++trial) {
        const int bs = 1 + (int)(rnd() % 6), ld = 15;
        std::vector<int32_t> lens(bs), alloc(bs), total(1);
        std::vector<double> S(bs * ld, 0.0);
        std::vector<int64_t> rb(bs);
        std::vector<uint32_t> fl(bs, 0);
        for (int r = 0; r < bs; ++r) {
            int32_t d[7], g[15], tok[15], src;
            double c[7], h[15];
            uint8_t f[15];
            int near;
            for (int k = 0; k < 7; ++k) { d[k] = (int32_t)(rnd() % 4); c[k] = urand(); }
            const int glen = (int)(rnd() % 16);
            for (int k = 0; k < glen; ++k) { g[k] = (int32_t)(rnd() % 4); h[k] = urand(); }
            lens[r] = oracle_select(7, d, c, 7, g, h, glen, 0.3, (int)(rnd() % 5), (int)(rnd() % 2), ld, tok, f,
                                    &S[r * ld], &src, &near);
            CHECK(lens[r] >= 0 && lens[r] <= ld);
        }
        oracle_allocate(bs, ld, lens.data(), S.data(), (int)(rnd() % 40), alloc.data(), rb.data(), total.data(),
                        fl.data());
        for (int r = 0; r < bs; ++r) CHECK(alloc[r] >= 0 && alloc[r] <= lens[r]);
    }
    // chain verification at T = 0 and T > 0
    {
        const int bs = 3, V = 50, ld = 4;
        std::vector<float> z(bs * (ld + 1) * V), w(bs * ld * V);
        for (auto& x : z) x = (float)(urand() * 4 - 2);
        for (auto& x : w) x = (float)(urand() * 4 - 2);
        std::vector<int64_t> rb = {0, ld + 1, 2 * (ld + 1)}, drb = {0, ld, 2 * ld};
        std::vector<int32_t> tok(bs * ld), ns = {ld, 2, 0}, ot(bs * (ld + 1)), on(bs), oa(bs), lo(bs), hi(bs);
        for (auto& x : tok) x = (int32_t)(rnd() % V);
        tok[1] = V + 3;   // an out-of-range token
        std::vector<uint8_t> sf(bs * ld, 0);
        std::vector<float> ua(bs * ld), us(bs);
        for (auto& x : ua) x = (float)urand();
        for (auto& x : us) x = (float)urand();
        std::vector<double> op(bs * (ld + 1)), oq(bs * ld);
        for (double T : {0.0, 0.7, 1.0}) {
            std::vector<uint32_t> fl(bs, 0);
            oracle_verify_chain(bs, V, T, z.data(), 0, V, rb.data(), w.data(), 0, V, drb.data(), tok.data(),
                                sf.data(), ld, ns.data(), ua.data(), us.data(), ot.data(), on.data(), oa.data(),
                                op.data(), oq.data(), fl.data(), lo.data(), hi.data());
            for (int r = 0; r < bs; ++r) {
                CHECK(on[r] == oa[r] + 1);
                CHECK(lo[r] <= ot[r * (ld + 1) + oa[r]] && ot[r * (ld + 1) + oa[r]] <= hi[r]);
            }
        }
    }
    // rows from caller-built forests, broken ones included
    for (int trial = 0; trial < 300; ++trial) {
        const int c_max = 1 + (int)(rnd() % 80), rows_cap = 1 + (int)(rnd() % 64);
        const int n = (int)(rnd() % (c_max + 3)) - 1;
        std::vector<int32_t> tok(c_max), par(c_max, -1), nt(rows_cap), pr(rows_cap), nr(1);
        std::vector<float> q(c_max, 0.0f);
        std::vector<double> Q(rows_cap), Sc(rows_cap), fQ(c_max);
        for (int j = 1; j < c_max; ++j) {
            tok[j] = (int32_t)(rnd() % 9);
            par[j] = (int32_t)(rnd() % j);
            q[j] = (float)urand();
        }
        if (trial % 7 == 0 && c_max > 2) par[1 + rnd() % (c_max - 1)] = c_max + 5;
        if (trial % 11 == 0 && c_max > 2) q[1 + rnd() % (c_max - 1)] = NAN;
        uint32_t fl = 0;
        const int used = oracle_tree_forest(n, c_max, tok.data(), par.data(), q.data(), rows_cap, nt.data(), pr.data(),
                                            Q.data(), nr.data(), Sc.data(), fQ.data(), &fl);
        CHECK(used >= 1 && used <= c_max && nr[0] >= 1 && nr[0] <= rows_cap && nr[0] <= used);
        for (int i = 1; i < nr[0]; ++i) CHECK(pr[i] >= 0 && pr[i] < i && Q[i] <= Q[pr[i]]);
    }
    // Philox4x32-10 known-answer vector of its authors (counter and key all zero)
    {
        const uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0};
        uint32_t out[4];
        oracle_philox4x32_10(ctr, key, out);
        CHECK(out[0] == 0x6627e8d5u && out[1] == 0xe169c58du && out[2] == 0xbc57ac4cu && out[3] == 0x9b00dbd8u);
    }
    return 0;
}

int main()
{
    int rc = budget_sizing();
    if (!rc) rc = validation();
    if (!rc) rc = oracle_functions();
    printf(rc ? "host checks FAILED\n" : "host checks passed\n");
    return rc;
}
