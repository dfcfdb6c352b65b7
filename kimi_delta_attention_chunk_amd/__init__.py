"""MI355X (gfx950) chunked forward of Kimi Delta Attention (KDA).

The computation runs in hand-written HIP kernels behind the C ABI of include/kda.h; this
package only loads that library (libkda.so, built in-tree) and marshals torch tensors.
"""
from .ops import (  # noqa: F401
    KdaError,
    chunk_fwd,
    kda_chunk_fwd,
    kda_chunk_fwd_plan,
    kda_chunk_fwd_plan_kernels,
    kda_kernel_variants,
    kda_chunk_fwd_workspace,
    kda_num_stages,
    kda_stage_name,
    kda_status_str,
    make_shape,
)

__all__ = ["KdaError", "chunk_fwd", "kda_chunk_fwd", "kda_chunk_fwd_plan", "kda_chunk_fwd_plan_kernels", "kda_kernel_variants",
           "kda_chunk_fwd_workspace", "kda_num_stages", "kda_stage_name", "kda_status_str", "make_shape"]
