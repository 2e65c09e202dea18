"""Medusa speculate-and-verify step on AMD MI355X (gfx950).

The verify step runs in libmedusa.so, a C-ABI library of hand-written HIP
kernels (``include/medusa.h``).  This package is its Python binding: the
functions below carry the C entry points' names and only marshal torch
tensors (device memory, the current stream) into those calls.

Build the library in-tree with ``python speculative_decoding_medusa_amd/build.py``;
importing the package without it raises ImportError.
"""

from ._lib import (  # noqa: F401
    MEDUSA_BF16, MEDUSA_F32, SPEC_STATUS, EXPORTED, LIB_PATH, MedusaError, lib, workspace,
    medusa_heads_workspace, medusa_resblock, medusa_lm_head_topk, medusa_heads, medusa_heads_noalloc, medusa_heads_tree,
    medusa_lm_head_topk_tree,
    medusa_build_tree,
    medusa_heads_pack, medusa_lm_head_topk_packed, medusa_heads_packed, medusa_tree_candidates,
    medusa_linear_workspace, medusa_linear,
    medusa_tree_attention_workspace, medusa_tree_attention, medusa_posterior_workspace,
    medusa_evaluate_posterior, medusa_posterior_nucleus_workspace, medusa_evaluate_posterior_nucleus,
    medusa_commit_kv, medusa_base_lm_head, medusa_base_lm_head_pack,
    medusa_base_posterior_workspace, medusa_base_posterior, medusa_embed, medusa_add_rmsnorm, medusa_rope_qkv,
    medusa_silu_mul, medusa_philox_uniforms, medusa_sample_typical, PURPOSE_NUCLEUS, PURPOSE_NEXT_TOKEN,
)

__all__ = [
    "MEDUSA_BF16", "MEDUSA_F32", "SPEC_STATUS", "MedusaError", "workspace",
    "medusa_heads_workspace", "medusa_resblock", "medusa_lm_head_topk", "medusa_heads", "medusa_heads_noalloc",
    "medusa_heads_tree", "medusa_lm_head_topk_tree",
    "medusa_heads_pack",
    "medusa_lm_head_topk_packed", "medusa_heads_packed", "medusa_tree_candidates", "medusa_linear_workspace",
    "medusa_linear",
    "medusa_build_tree", "medusa_tree_attention_workspace", "medusa_tree_attention",
    "medusa_posterior_workspace", "medusa_evaluate_posterior", "medusa_posterior_nucleus_workspace",
    "medusa_evaluate_posterior_nucleus", "medusa_commit_kv", "medusa_base_lm_head",
    "medusa_base_lm_head_pack", "medusa_base_posterior_workspace", "medusa_base_posterior",
    "medusa_embed", "medusa_add_rmsnorm", "medusa_rope_qkv", "medusa_silu_mul",
    "medusa_philox_uniforms", "medusa_sample_typical", "PURPOSE_NUCLEUS", "PURPOSE_NEXT_TOKEN",
]
