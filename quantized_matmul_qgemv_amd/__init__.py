"""Weight-quantized GEMV / GEMM / grouped-MoE GEMM for MI355X (gfx950).

The compute path is libqmm.so (hand-written HIP kernels behind the C ABI in
include/qmm.h); this package only marshals torch device tensors into it.
"""
from ._lib import QmmError, lib, last_error  # noqa: F401
from .api import (  # noqa: F401
    GemmBatchPlan, GemvPlan, convert_bf16, dequant, moe_combine, moe_gate_up_swiglu, moe_plan_dropped,
    moe_route, moe_route_size, qgemm, qgemm_batched, qgemm_batched_plan, qgemm_grouped,
    qgemm_grouped_noalloc,
    qgemm_grouped_workspace_size,
    qgemm_workspace_size, qgemv, qgemv_batched, qgemv_batched_plan, quantize, repack_scales_tiled,
    repack_tiled, unpack_codes,
)

__all__ = [
    "QmmError", "lib", "last_error", "GemmBatchPlan", "GemvPlan", "dequant", "qgemm",
    "convert_bf16", "moe_combine", "moe_gate_up_swiglu", "moe_plan_dropped", "moe_route",
    "moe_route_size", "qgemm_batched", "qgemm_grouped_noalloc", "qgemm_batched_plan", "qgemm_grouped",
    "qgemm_grouped_workspace_size", "qgemm_workspace_size", "qgemv", "qgemv_batched",
    "qgemv_batched_plan", "quantize", "repack_scales_tiled", "repack_tiled", "unpack_codes",
]
