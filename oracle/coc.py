"""Plain fp64 definitions of the fused matmul + collective ops, one rank's share.

Test infrastructure only (see oracle/__init__.py).

Pages cited (by title, section):
  * CoC guide -- Ascend PyTorch developer guide, MindSpeed page
    "Communication-over-Computation (计算通信并行)".
  * Overlap blog -- "MindSpeed LLM通信计算重叠与MC2如何榨干昇腾芯片算力".

What the ops compute (CoC guide, "Problem analysis" and "Approach - fused-kernel
implementation"): the ColumnParallelLinear / RowParallelLinear matmul and the
tensor-parallel collective that follows or precedes it.  Without sequence
parallelism a RowParallel matmul is followed by an AllReduce of the per-rank
partial products; with sequence parallelism the RowParallel matmul is followed
by a ReduceScatter and the ColumnParallel matmul is preceded by an AllGather.
Splitting the left matrix along m into 2/4/8 pieces only reorders the work,
so none of the definitions below depends on the split count.

Conventions (all readings, since the pages give no layout):
  * X is m x k, W is k x n, Y is m x n, all row-major, rank rho in [0, T).
  * ``peers[r]`` for r != rho is the partial product peer r contributes; the
    entry at index rho is ignored (this rank's own partial is X @ W).
  * Reduce-scatter and all-gather act on rows (the sequence dimension):
    rank r owns rows [r*m/T, (r+1)*m/T).
  * All inputs are values of the storage dtype, passed here as float64 arrays;
    products of two such values are exact in float64, so the float64 results
    are the exact real results up to float64 summation error (k * 2**-53).
"""
from __future__ import annotations

import numpy as np

from .formats import round_dtype


def matmul(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """P = X @ W in float64 (the "Matmul" half of every pair)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[0]:
        raise ValueError(f"matmul shapes {x.shape} @ {w.shape}")
    return x @ w


def _peer_sum(peers, rank: int, rows=None) -> np.ndarray | None:
    acc = None
    for r, p in enumerate(peers):
        if r == rank:
            continue
        p = np.asarray(p, dtype=np.float64)
        if rows is not None:
            p = p[rows]
        acc = p.copy() if acc is None else acc + p
    return acc


def matmul_all_reduce(x, w, peers, rank: int):
    """MATMUL_ALL_REDUCE (CoC guide, fused-operator list; compute, then communicate).

    Returns (Y, P): P = X @ W is this rank's partial product, and
    Y = P + sum over r != rank of peers[r], the all-reduced output.
    """
    p = matmul(x, w)
    s = _peer_sum(peers, rank)
    y = p.copy() if s is None else p + s
    return y, p


def matmul_reduce_scatter(x, w, peers, rank: int, rows=None):
    """MATMUL_REDUCE_SCATTER (CoC guide, fused-operator list; compute, then communicate).

    T = len(peers).  Rank ``rank`` receives rows [rank*m/T, (rank+1)*m/T) of
    the all-reduced product.  Returns (Y_slice, P) with P = X @ W over all m
    rows (the partial this rank hands to the others).

    ``rows`` (optional) restricts the evaluation to local slice rows
    ``rows`` (indices into the m/T-row slice); P is then only evaluated on
    those rows as well.
    """
    x = np.asarray(x, dtype=np.float64)
    T = len(peers)
    m = x.shape[0]
    if m % T:
        raise ValueError("m must be a multiple of the world size")
    b = m // T
    local = np.arange(b) if rows is None else np.asarray(rows)
    glob = rank * b + local
    p_rows = matmul(x[glob], w)
    s = _peer_sum(peers, rank, glob)
    y = p_rows.copy() if s is None else p_rows + s
    p = matmul(x, w) if rows is None else p_rows
    return y, p


def allgather(shards) -> np.ndarray:
    """AllGather along rows: block r of the result is rank r's shard."""
    return np.vstack([np.asarray(s, dtype=np.float64) for s in shards])


def allgather_matmul(shards, w):
    """ALL_GATHER_MATMUL and ALL_GATHER_MATMUL_V2 (CoC guide, fused-operator list).

    Communicate, then compute: G = vstack(shards), Y = G @ W.  The V2 form
    also hands back G, so both are returned as (Y, G).
    """
    g = allgather(shards)
    return matmul(g, w), g


def weight_grad(g, dy) -> np.ndarray:
    """Weight gradient of the sequence-parallel pair (CoC guide, "Approach":
    the fused operators come in forward / backward pairs, and V2 hands back the
    all-gathered G so the backward pass can reuse it): dW = G^T @ dY in
    float64, G m x k, dY m x n, dW k x n."""
    g = np.asarray(g, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    if g.ndim != 2 or dy.ndim != 2 or g.shape[0] != dy.shape[0]:
        raise ValueError(f"shape mismatch {g.shape} {dy.shape}")
    return g.T @ dy


def dequant_weight(q, scales, mode: str, group: int = 0) -> np.ndarray:
    """Weight-only int8 dequantisation for w8A16 (CoC guide, last item of the
    fused-operator list: per tensor, per channel, per group).

    Reading: symmetric, no zero point, W~[k, n] = q[k, n] * s with
      per_tensor : s = scales[0]
      per_channel: s = scales[n]                 (one scale per output column)
      per_group  : s = scales[k // group, n]     (groups run along K)
    The product of an int8 and an fp16 value is exact in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    K, N = q.shape
    if mode == "per_tensor":
        return q * s.reshape(-1)[0]
    if mode == "per_channel":
        return q * s.reshape(1, N)
    if mode == "per_group":
        if group <= 0 or K % group:
            raise ValueError("per_group needs K divisible by the group size")
        s = s.reshape(K // group, N)
        return q * np.repeat(s, group, axis=0)
    raise ValueError(f"unknown quant mode {mode}")


def matmul_all_reduce_w8a16(x, q, scales, mode: str, group: int, peers, rank: int):
    """w8A16 MATMUL_ALL_REDUCE: fp16 activations times the dequantised int8 weight,
    then the all-reduce of the partials.  Returns (Y, P)."""
    return matmul_all_reduce(x, dequant_weight(q, scales, mode, group), peers, rank)


def reduce_fixed_order(partials, dtype: str) -> np.ndarray:
    """Deterministic sum of stored partials (CoC guide: the deterministic variants
    of MATMUL_ALL_REDUCE and MATMUL_REDUCE_SCATTER).

    The pages do not fix the order or the accumulator.  Reading: every rank
    adds the stored partials in ascending rank order 0..T-1 in binary32, each
    addition rounded to nearest-even, and rounds the sum once to ``dtype``;
    this rank's own partial takes part as stored (rounded to ``dtype``), so
    every rank obtains the same bits.
    """
    acc = None
    for p in partials:
        v = np.asarray(p, dtype=np.float64).astype(np.float32)
        acc = v.copy() if acc is None else (acc + v)     # binary32 add, RNE
    return round_dtype(acc.astype(np.float64), dtype)


def normwise_rel_error(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64 (0 when both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
