"""MI355X (gfx950) speculative-decoding step: n-gram draft, verification-budget
allocation (with host budget sizing), lossless chain verification and greedy tree
verification.

The compute lives in ``libspec_hip.so`` (hand-written HIP kernels behind the C
ABI of include/spec.h); this package is its thin binding.
"""
from ._lib import (  # noqa: F401
    FLAG_BAD_LENGTH,
    FLAG_BAD_LOGITS,
    FLAG_BAD_TOKEN,
    FLAG_CTX_OVERFLOW,
    FLAG_RESIDUAL_LATE,
    FLAG_RESIDUAL_ZERO,
    LIB_PATH,
    POLICIES,
    spec_allocate_budget,
    spec_ngram_draft,
    spec_size_budget,
    spec_verify_chain,
    spec_verify_tree,
)
from . import _lib  # noqa: F401
