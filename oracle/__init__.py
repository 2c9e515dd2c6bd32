"""CPU oracle for the fused matmul + tensor-parallel collective ops.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library path never does,
and this package imports nothing from the library.  It computes, in float64
and in the plainest form, what each op is defined to produce, so that the HIP
path can be checked against it.

Pinning: every function here is checked in tests/test_oracle_*.py against
something other than itself (closed forms, brute force with exact rationals,
library conversions, invariants); see the docstrings there.
"""
from .formats import round_to, encode, decode, round_f32, round_dtype, decode_dtype
from .coc import (
    matmul,
    matmul_all_reduce,
    matmul_reduce_scatter,
    allgather,
    allgather_matmul,
    weight_grad,
    dequant_weight,
    matmul_all_reduce_w8a16,
    reduce_fixed_order,
    normwise_rel_error,
)
from .moe import (
    received_order,
    alltoall_dispatch,
    group_rows,
    grouped_matmul,
    alltoall_grouped_matmul,
    alltoall_combine,
    grouped_matmul_alltoall,
)

__all__ = [
    "round_to", "encode", "decode", "round_f32", "round_dtype", "decode_dtype",
    "matmul", "matmul_all_reduce", "matmul_reduce_scatter", "allgather",
    "allgather_matmul", "weight_grad", "dequant_weight", "matmul_all_reduce_w8a16",
    "reduce_fixed_order", "normwise_rel_error",
    "received_order", "alltoall_dispatch", "group_rows", "grouped_matmul",
    "alltoall_grouped_matmul", "alltoall_combine", "grouped_matmul_alltoall",
]
