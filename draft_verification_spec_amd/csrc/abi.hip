// C-ABI entry points: argument validation, workspace sizing, dispatch.
// Every host-detectable error returns before anything is enqueued.
#include <string.h>

#include "common.hpp"

size_t spec_ngram_ws(const spec_ngram_args* a);
int spec_ngram_launch(const spec_ngram_args* a, hipStream_t st);
size_t spec_alloc_ws(const spec_alloc_args* a);
int spec_alloc_launch(const spec_alloc_args* a, hipStream_t st);
size_t spec_verify_chain_ws(int32_t bs, int32_t vocab, int32_t ld, int32_t dtype);
int spec_verify_chain_launch(const spec_verify_args* a, hipStream_t st);
int spec_verify_chain_noalloc_launch(const spec_verify_args* a, hipStream_t st);
size_t spec_verify_tree_ws(int32_t bs, int32_t vocab, int32_t rows_max, int32_t dtype);
int spec_verify_tree_launch(const spec_tree_verify_args* a, hipStream_t st);

static thread_local char g_hip_error[256] = "";

int spec_record_hip_error(hipError_t e)
{
    if (e == hipSuccess) return SPEC_OK;
    const char* s = hipGetErrorString(e);
    strncpy(g_hip_error, s ? s : "unknown HIP error", sizeof(g_hip_error) - 1);
    g_hip_error[sizeof(g_hip_error) - 1] = 0;
    return SPEC_EHIP;
}

#include "validate.hpp"

using namespace spec_validate;

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_strerror(int code)
{
    switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SPEC_EHIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

const char* spec_last_hip_error(void) { return g_hip_error; }

size_t spec_workspace_bytes(int op, const void* args)
{
    if (!args) return 0;
    switch (op) {
    case SPEC_OP_NGRAM: {
        const spec_ngram_args* a = (const spec_ngram_args*)args;
        return check_ngram(a) == SPEC_OK ? spec_ngram_ws(a) : 0;
    }
    case SPEC_OP_ALLOCATE: {
        const spec_alloc_args* a = (const spec_alloc_args*)args;
        return check_alloc(a) == SPEC_OK ? spec_alloc_ws(a) : 0;
    }
    case SPEC_OP_VERIFY_CHAIN: {
        const spec_verify_args* a = (const spec_verify_args*)args;
        return check_verify(a) == SPEC_OK ? spec_verify_chain_ws(a->bs, a->vocab, a->ld, a->dtype) : 0;
    }
    case SPEC_OP_VERIFY_TREE: {
        const spec_tree_verify_args* a = (const spec_tree_verify_args*)args;
        return check_tree_verify(a) == SPEC_OK ? spec_verify_tree_ws(a->bs, a->vocab, a->rows_max, a->dtype) : 0;
    }
    default: return 0;
    }
}

int spec_ngram_draft(const spec_ngram_args* a, void* stream)
{
    int rc = check_ngram(a);
    if (rc) return rc;
    rc = check_workspace(a->workspace, a->workspace_bytes, spec_ngram_ws(a));
    if (rc) return rc;
    if (a->nq == 0) return SPEC_OK;
    return spec_ngram_launch(a, (hipStream_t)stream);
}

int spec_allocate_budget(const spec_alloc_args* a, void* stream)
{
    int rc = check_alloc(a);
    if (rc) return rc;
    rc = check_workspace(a->workspace, a->workspace_bytes, spec_alloc_ws(a));
    if (rc) return rc;
    return spec_alloc_launch(a, (hipStream_t)stream);
}

int spec_verify_chain(const spec_verify_args* a, void* stream)
{
    int rc = check_verify(a);
    if (rc) return rc;
    rc = check_workspace(a->workspace, a->workspace_bytes, spec_verify_chain_ws(a->bs, a->vocab, a->ld, a->dtype));
    if (rc) return rc;
    return spec_verify_chain_launch(a, (hipStream_t)stream);
}

int spec_verify_chain_noalloc(const spec_verify_args* a, void* stream)
{
    int rc = check_verify(a);
    if (rc) return rc;
    return spec_verify_chain_noalloc_launch(a, (hipStream_t)stream);
}

int spec_verify_tree(const spec_tree_verify_args* a, void* stream)
{
    int rc = check_tree_verify(a);
    if (rc) return rc;
    rc = check_workspace(a->workspace, a->workspace_bytes, spec_verify_tree_ws(a->bs, a->vocab, a->rows_max, a->dtype));
    if (rc) return rc;
    return spec_verify_tree_launch(a, (hipStream_t)stream);
}

}  // extern "C"
