// Host-side argument validation of the C ABI (include/spec.h): plain C++
// over the argument structs, with no HIP dependency, so that it also builds
// into host-only test programs (the sanitizer build of the test suite).
// Every check returns SPEC_OK or SPEC_EINVAL / SPEC_EWORKSPACE and touches
// no device memory.
#pragma once

#include <stdint.h>

#include "spec.h"

namespace spec_validate {

#define REQUIRE(c) \
    do {           \
        if (!(c)) return SPEC_EINVAL; \
    } while (0)

inline int check_ngram(const spec_ngram_args* a)
{
    REQUIRE(a);
    REQUIRE(a->bs >= 1 && a->nq >= 0);
    REQUIRE(a->ctx && a->ctx_len && a->ctx_stride >= 1);
    REQUIRE(a->query_req || a->nq <= a->bs);
    REQUIRE(!a->extra || (a->extra_len && a->extra_stride >= 0));
    REQUIRE(a->ctx_stride + (a->extra ? a->extra_stride : 0) < ((int64_t)1 << 31));
    REQUIRE(a->n_min >= 1 && a->n_max >= a->n_min);
    REQUIRE(a->max_draft >= 1 && a->max_draft <= SPEC_MAX_DRAFT);
    REQUIRE(a->copy_cap >= a->n_min && a->copy_cap <= SPEC_MAX_CAP);
    REQUIRE(a->nq == 0 || (a->draft && a->draft_len && a->feat));
    REQUIRE(a->follow_ctx >= 0 && a->follow_ctx <= SPEC_MAX_FOLLOW_CTX);
    return SPEC_OK;
}

inline int check_chain_alloc(const spec_chain_alloc* c)
{
    REQUIRE(c->bs >= 1 && c->bs < (1 << 27) - 1);
    REQUIRE(c->ld >= 1 && c->ld <= SPEC_MAX_DRAFT);
    REQUIRE(c->K >= 0 && c->K <= c->ld);
    REQUIRE(c->ngram_ld >= 0 && c->ngram_ld <= c->ld);
    REQUIRE(c->K == 0 || (c->model_tokens && c->model_conf));
    REQUIRE(c->ngram_draft && c->ngram_len && c->ngram_feat);
    REQUIRE(c->budget >= 0);
    REQUIRE(c->policy >= SPEC_POLICY_PROPOSED && c->policy <= SPEC_POLICY_NGRAM_ONLY);
    REQUIRE(c->lambda == c->lambda);
    REQUIRE(c->chain_tokens && c->slot_flags && c->chain_len && c->chain_src && c->survival);
    REQUIRE(c->alloc_len && c->row_base && c->total_rows && c->out_flags);
    return SPEC_OK;
}

inline int check_tree_alloc(const spec_tree_alloc* t)
{
    REQUIRE(t->bs >= 1);
    REQUIRE(t->rows_cap >= 1 && t->rows_cap <= SPEC_MAX_ROWS);
    REQUIRE(t->node_token && t->parent_row && t->Q && t->n_rows && t->row_base && t->total_rows);
    REQUIRE(t->forest_count && t->out_flags);
    if (t->forest_token) {   // a caller-built forest
        REQUIRE(t->forest_parent && t->forest_q && t->forest_n && !t->scores);
        REQUIRE(t->c_max >= 1 && t->c_max <= SPEC_MAX_FOREST);
        return SPEC_OK;
    }
    REQUIRE(t->P >= 0 && t->Kc >= 1);
    REQUIRE(t->P == 0 || t->block);
    REQUIRE(t->c_max >= 1 + t->P * t->Kc && t->c_max <= SPEC_MAX_FOREST);
    REQUIRE(t->ngram_ld >= 0 && (t->ngram_ld == 0 || t->ngram_draft) && t->ngram_len);
    REQUIRE(t->scores || (t->w_node && t->w_none));
    if (t->scores) {
        const spec_tree_scores* sc = t->scores;
        REQUIRE(t->P == 0 || (sc->h && sc->sigma && (t->Kc == 1 || sc->r_share)));
        REQUIRE(sc->psi_ctx && sc->b_req && sc->p_src && sc->ngram_feat);
    }
    REQUIRE(t->depth_max >= 1);
    return SPEC_OK;
}

inline int check_alloc(const spec_alloc_args* a)
{
    REQUIRE(a);
    if (a->mode == SPEC_ALLOC_CHAIN) return check_chain_alloc(&a->chain);
    if (a->mode == SPEC_ALLOC_TREE) return check_tree_alloc(&a->tree);
    return SPEC_EINVAL;
}

inline bool dtype_ok(int dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

inline int check_verify(const spec_verify_args* a)
{
    REQUIRE(a);
    REQUIRE(a->bs >= 1 && a->vocab >= 1 && a->vocab <= SPEC_MAX_VOCAB);
    REQUIRE(a->temperature >= 0.0f && a->temperature < 1e30f);
    REQUIRE(a->logits && a->row_base && dtype_ok(a->dtype) && a->row_stride >= a->vocab && a->n_logit_rows >= 1);
    if (a->draft_logits) {
        REQUIRE(a->draft_row_base && dtype_ok(a->draft_dtype));
        REQUIRE(a->draft_row_stride >= a->vocab && a->n_draft_rows >= 1);
    }
    REQUIRE(a->tokens && a->n_slots && a->ld >= 1 && a->ld <= SPEC_MAX_DRAFT && a->max_slots >= 0);
    REQUIRE(a->temperature == 0.0f || a->rng || (a->u_accept && a->u_sample));
    REQUIRE(a->rng == 0 || a->rng == 1);
    REQUIRE(a->out_tokens && a->out_num && a->out_accepted && a->out_flags);
    if (a->ctx) REQUIRE(a->ctx_len && a->ctx_cap >= 0 && a->ctx_cap <= a->ctx_stride);
    if (a->ngram_draft) {
        REQUIRE(a->ctx && a->ctx_stride >= 1 && a->ctx_stride < ((int64_t)1 << 31));
        REQUIRE(a->ngram_draft_len && a->ngram_feat);
        REQUIRE(a->ngram_n_min >= 1 && a->ngram_n_max >= a->ngram_n_min);
        REQUIRE(a->ngram_max_draft >= 1 && a->ngram_max_draft <= SPEC_MAX_DRAFT);
        REQUIRE(a->ngram_copy_cap >= a->ngram_n_min && a->ngram_copy_cap <= SPEC_MAX_CAP);
    }
    return SPEC_OK;
}

inline int check_tree_verify(const spec_tree_verify_args* a)
{
    REQUIRE(a);
    REQUIRE(a->bs >= 1 && a->vocab >= 1 && a->vocab <= SPEC_MAX_VOCAB);
    REQUIRE(a->rows_max >= 1 && a->rows_max <= SPEC_MAX_ROWS);
    REQUIRE(a->logits && a->row_base && dtype_ok(a->dtype) && a->row_stride >= a->vocab && a->n_logit_rows >= 1);
    REQUIRE(a->node_token && a->parent_row && a->n_rows);
    REQUIRE(a->out_tokens && a->out_num && a->out_path_rows && a->out_flags);
    if (a->ctx) REQUIRE(a->ctx_len && a->ctx_cap >= 0 && a->ctx_cap <= a->ctx_stride);
    return SPEC_OK;
}

inline int check_workspace(void* ws, size_t have, size_t need)
{
    if (need == 0) return SPEC_OK;
    if (!ws || have < need) return SPEC_EWORKSPACE;
    if ((uintptr_t)ws % 256 != 0) return SPEC_EWORKSPACE;
    return SPEC_OK;
}


}  // namespace spec_validate
