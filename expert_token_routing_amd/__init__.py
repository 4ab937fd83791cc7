"""One expert-parallel rank's share of an MoE layer on AMD Instinct MI355X.

Route (router logits, top-k, combine weights) -> dispatch (rows grouped by
local expert) -> grouped SwiGLU expert MLPs -> combine (weighted sum in the
original token order), all in hand-written gfx950 HIP kernels behind the
C-ABI of ``include/moe.h``; this package is its Python binding.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK,
    NOALLOC_SCRATCH_BYTES, SIGNATURES,
    MoEError, check, forward_workspace_layout, forward_workspace_size, lib, moe_combine, moe_combine_f32, moe_dispatch,
    moe_expert_ffn, moe_forward, moe_forward_f32, moe_forward_fused, moe_forward_noalloc, moe_forward_profiled, moe_route,
    status_string,
)
