"""Absorbed Multi-head Latent Attention over a paged latent KV cache for MI355X (gfx950).

The compute lives in libmla.so (hand-written HIP kernels behind the C
interface in include/mla.h); this package is its thin Python binding plus
the seeded synthetic workload generator.
"""

from ._lib import (  # noqa: F401
    D_C, D_NOPE, D_R, D_V, MLA_BF16, MLA_ERR_HIP, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE,
    MLA_F32, MLA_FP8_E4M3, MLA_OK, PAGE, ROW, MLAError, PagedCache, absorb_q, cache_write, decode, decode_merge,
    decode_merge_upproj, decode_multi, decode_multi_upproj, decode_noalloc, decode_partial, decode_workspace,
    decode_upproj, decode_upproj_workspace, decode_upproj_launches, NOALLOC_SCRATCH_BYTES,
    decode_workspace_size, default_softmax_scale, lib, prefill_causal, status_string, upproj_v, MlaRope, yarn_rope,
    yarn_attention_factor, linear, linear_workspace_size, kv_append, kv_append_workspace_size, q_project,
    q_project_workspace_size, qkv_project, qkv_project_workspace_size, output_proj, fold_wuv_wo, set_debug, validate_decode_inputs,
)
