"""Fused Mixture-of-Experts layer forward for AMD MI355X (gfx950).

The compute path is the HIP library libmoemi.so with the C ABI of
``include/moe.h``; this package is its thin Python binding (``binding``), the
ahead-of-time build (``build``) and the seeded synthetic workloads
(``workloads``).  The library is loaded on first use; there is no fallback.
"""

from .binding import (  # noqa: F401
    FusedLayout,
    FusedMoE,
    NO_SECTION,
    WorkspacePool,
    MoEError,
    act_quant_fp8,
    act_quant_fp8_rows,
    align,
    align_capacity,
    fused_block_m,
    fused_forward,
    fused_forward_noalloc,
    inv_rope_fp8_quant_per_head,
    lib,
    route_topk,
)
