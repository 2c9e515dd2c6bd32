"""Seeded synthetic inputs for the fused matmul + collective ops.

This module only draws random numbers and stores them in the op's dtype; it
holds none of the ops' arithmetic and imports nothing else from this
package, so the tests can feed the same inputs to the library and to the
CPU oracle.

Seeds: ``numpy.random.SeedSequence([0, workload, tensor, rank])``.
Storage conversion goes through torch (float32 -> bfloat16 / float16 round
to nearest even) or numpy (float -> float16, int8).

Workloads: one tensor-parallel rank (world 8) of the RowParallel /
ColumnParallel linears of three model shapes the CoC guide's results section
names (BLOOM 7B, BLOOM 176B, LLaMA2 70B), plus a small fp32 case.  Weights and
activations are random (N(0,1) activations, N(0, 0.02^2) weights); the other
ranks' partial sums are random with the standard deviation a real partial of
that shape would have, sqrt(k) * 1 * 0.02 (w8a16: sqrt(k) * rms(q * scale)).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids
T_X, T_W, T_PEER, T_PEER_W, T_SCALES = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    op: str                 # all_reduce | reduce_scatter | allgather | w8a16
    dtype: str              # f32 | f16 | bf16
    m: int
    n: int
    k: int
    world: int
    splits: tuple
    det: tuple = (0, 1)
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    peer_sigma: float = 1.0
    group: int = 128
    note: str = ""


WORKLOADS = {
    "toy_f32": Workload("toy_f32", 0, "all_reduce", "f32", 256, 256, 256, 2, (2,),
                        note="X 256x512, W 512x256 uniform[-1,1]; rank 0 holds K shard 0 (256), "
                             "the peer partial is the K shard 1 product"),
    "bloom7b_ar": Workload("bloom7b_ar", 1, "all_reduce", "bf16", 2048, 4096, 2048, 8, (4, 2, 8),
                           peer_sigma=0.905, note="BLOOM-7B down-proj, TP8 rank"),
    "llama70b_ag": Workload("llama70b_ag", 2, "allgather", "bf16", 4096, 7168, 8192, 8, (4, 8),
                            note="LLaMA2-70B fused gate/up, TP8+SP: 8 shards of 512x8192"),
    "llama70b_rs": Workload("llama70b_rs", 3, "reduce_scatter", "bf16", 4096, 8192, 3584, 8, (4, 8),
                            peer_sigma=1.197, note="LLaMA2-70B down-proj, TP8+SP"),
    "bloom176b_ar": Workload("bloom176b_ar", 4, "all_reduce", "bf16", 2048, 14336, 7168, 8, (2, 4, 8),
                             det=(1,), peer_sigma=1.693, note="BLOOM-176B down-proj, deterministic"),
    "w8a16_ar": Workload("w8a16_ar", 5, "w8a16", "f16", 4096, 8192, 3584, 8, (4,),
                         peer_sigma=52.0, note="int8 weights, fp16 scales in [0.001, 0.02]"),
}


def rng_for(wid: int, tensor: int, rank: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, wid, tensor, rank]))


def _to_torch(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "f32":
        return t.to(torch.float32)
    if dtype == "bf16":
        return t.to(torch.float32).to(torch.bfloat16)
    if dtype == "f16":
        return t.to(torch.float32).to(torch.float16)
    if dtype == "i8":
        return t.to(torch.int8)
    raise ValueError(dtype)


def normal(wid, tensor, rank, shape, sigma, dtype):
    """N(0, sigma^2) values stored in ``dtype`` (torch CPU tensor)."""
    g = rng_for(wid, tensor, rank)
    a = g.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return _to_torch(a, dtype)


def uniform(wid, tensor, rank, shape, lo, hi, dtype):
    g = rng_for(wid, tensor, rank)
    return _to_torch(g.uniform(lo, hi, shape).astype(np.float32), dtype)


def integers(wid, tensor, rank, shape, lo, hi, dtype):
    """Uniform integers in [lo, hi] stored in ``dtype`` (exact in every dtype used)."""
    g = rng_for(wid, tensor, rank)
    return _to_torch(g.integers(lo, hi + 1, shape).astype(np.float32 if dtype != "i8" else np.int8), dtype)


def fp16_scales(wid, rank, shape, lo=0.001, hi=0.02):
    g = rng_for(wid, T_SCALES, rank)
    import torch
    return torch.from_numpy(g.uniform(lo, hi, shape).astype(np.float16))


def pow2_scales(wid, rank, shape, lo_exp=-6, hi_exp=-2):
    """Scales 2^e, e uniform in [lo_exp, hi_exp]: products with small ints stay exact."""
    g = rng_for(wid, T_SCALES, rank)
    import torch
    e = g.integers(lo_exp, hi_exp + 1, shape)
    return torch.from_numpy(np.ldexp(1.0, e).astype(np.float16))


def peers_random(wid, world, rank, shape, sigma, dtype):
    """The other ranks' partials as random draws; entry ``rank`` is None."""
    return [None if r == rank else normal(wid, T_PEER, r, shape, sigma, dtype) for r in range(world)]


# ------------------------------------------------------------------ MoE expert all-to-all
# One expert-parallel rank of a MoE layer: every source rank of the group
# routes each of its tokens to top-k distinct experts drawn uniformly (the
# routing itself is input here, not part of the op), its tokens cut into
# `pieces` equal sequence pieces.  Rows and weights are N(0,1) and N(0, 0.02^2).
T_ROUTE, T_SEND, T_EXPERT_W = 5, 6, 7


@dataclass(frozen=True)
class MoeWorkload:
    name: str
    wid: int
    dtype: str
    world: int          # expert-parallel ranks
    experts: int        # experts in all (world * local)
    topk: int
    tokens: int         # tokens per source rank
    hidden: int         # k of the first matmul, n of the second
    ffn: int            # n of the first matmul, k of the second
    pieces: int
    rank: int = 0
    note: str = ""

    @property
    def local(self) -> int:
        return self.experts // self.world


MOE_WORKLOADS = {
    "moe_small": MoeWorkload("moe_small", 20, "bf16", 2, 4, 2, 512, 256, 384, 2, rank=1,
                             note="small case of the Ampipe scenario's routing (4 experts, top 2, EP 2)"),
    "moe_ragged": MoeWorkload("moe_ragged", 21, "f16", 8, 16, 2, 300, 128, 224, 4, rank=5,
                              note="EP 8, 2 local experts, ragged groups"),
    "moe_ampipe": MoeWorkload("moe_ampipe", 22, "bf16", 2, 4, 2, 8192, 12288, 49152, 2, rank=0,
                              note="Ampipe page scenario: hidden 12288, 4 experts, top 2, EP 2; "
                                   "sequence 128k over CP 2 and TP 8 (sequence parallel): 8192 tokens "
                                   "per rank; ffn 4 x hidden; Ampipe degree 2"),
}


def moe_counts(wl: MoeWorkload) -> np.ndarray:
    """counts[p][r][e]: rows source r routes to local expert e of rank wl.rank
    in sequence piece p (pieces: equal runs of the source's tokens)."""
    local = wl.local
    counts = np.zeros((wl.pieces, wl.world, local), dtype=np.int64)
    bounds = [wl.tokens * p // wl.pieces for p in range(wl.pieces + 1)]
    for r in range(wl.world):
        g = rng_for(wl.wid, T_ROUTE, r)
        choice = np.argsort(g.random((wl.tokens, wl.experts)), axis=1)[:, :wl.topk]
        for p in range(wl.pieces):
            sel = choice[bounds[p]:bounds[p + 1]].ravel() - wl.rank * local
            sel = sel[(sel >= 0) & (sel < local)]
            counts[p, r] = np.bincount(sel, minlength=local)
    return counts


def moe_sends(wl: MoeWorkload, counts: np.ndarray, width: int):
    """Each source's rows for this rank (rows x width, N(0,1)), CPU tensors."""
    return [normal(wl.wid, T_SEND, r, (int(counts[:, r, :].sum()), width), 1.0, wl.dtype)
            for r in range(wl.world)]


def moe_weights(wl: MoeWorkload, k: int, n: int, which: int = 0):
    """The local experts' weights, local x k x n, N(0, 0.02^2) (CPU tensor)."""
    return normal(wl.wid, T_EXPERT_W, which, (wl.local, k, n), 0.02, wl.dtype)
