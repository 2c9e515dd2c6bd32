"""Fused matmul + tensor-parallel collective ops for MI355X (gfx950).

The ops run in the HIP kernels of libcoc.so (C ABI in include/coc.h); this
package is its Python binding.  The library is loaded on first use.
"""
from .coc import (  # noqa: F401
    CocError,
    COC_F32, COC_F16, COC_BF16,
    COC_PER_TENSOR, COC_PER_CHANNEL, COC_PER_GROUP,
    OP_MATMUL_ALL_REDUCE, OP_MATMUL_REDUCE_SCATTER, OP_ALLGATHER_MATMUL,
    OP_ALLGATHER_MATMUL_V2, OP_MATMUL_ALL_REDUCE_W8A16,
    EXPORTS, LIB_PATH,
    lib,
    matmul_all_reduce,
    matmul_reduce_scatter,
    allgather_matmul,
    allgather_matmul_noalloc,
    matmul_all_reduce_w8a16,
    weight_grad,
    alltoall_grouped_matmul,
    grouped_matmul_alltoall,
    workspace_bytes,
    check_waits,
    plan,
    profile_enable,
    profile_stamps,
    profile_stamp_count,
    profile_read,
    profile_records,
    diag_mfma_loop,
)
