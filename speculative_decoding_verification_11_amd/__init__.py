"""Speculative-sampling verification on AMD Instinct MI355X (gfx950).

The hot path is the C-ABI HIP library declared in include/spec_verify.h;
``spec_verify``, ``spec_verify_early_exit``, ``spec_verify_top_p``,
``spec_verify_top_k_top_p``, ``spec_verify_tree`` and ``spec_prompt_lookup``
below are its thin Python
binding. ``workloads`` draws the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    BF16, F32, MAX_K, MAX_TREE, MAX_NGRAM, SpecVerifyError, spec_verify, spec_verify_early_exit,
    spec_verify_noalloc, NOALLOC_SCRATCH_BYTES,
    spec_verify_top_p, spec_verify_top_k_top_p, spec_verify_tree, spec_prompt_lookup, strerror,
    workspace_size, tree_workspace_size, library,
    SEQ_OK, SEQ_BAD_TOKEN, SEQ_BAD_LEN, SEQ_BAD_TEMP, SEQ_QZERO, SEQ_BAD_TREE, SEQ_BAD_TOP_P,
    DRAW_NONE, DRAW_GREEDY, DRAW_RESIDUAL, DRAW_BONUS, DRAW_RESIDUAL_AS_P,
)

__version__ = "0.1.0"
