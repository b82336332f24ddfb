"""Lighthouse attention layer for AMD Instinct MI355X (gfx950).

The work runs in liblh.so (HIP kernels behind the C ABI in include/lh_api.h); `ops` is the
thin Python binding with the C entry points' names, `synth` the seeded workload generator.
"""

from .ops import (  # noqa: F401
    Buffers, attn_desc, config_for, lh_attn_bwd, lh_attn_bwd_mapped, lh_attn_fwd,
    lh_attn_fwd_mapped, lh_backward, lh_build_map, lh_forward, lh_forward_noalloc, lh_gather,
    lh_gather_pool_bwd, lh_plan, lh_pool_score, lh_pool_score_topk, lh_scatter, lh_scatter_bwd,
    lh_status_string, lh_topk, make_config,
)
