"""The largest sizes the library accepts: one of m*n, m*k or k*n just below
2^31 elements (each byte offset of a bf16 matrix just below 4 GiB).  Inputs
are drawn on the GPU (integer-valued operands, so the matmul is exact in
binary32 and partial_out has one correct bit pattern); outputs are checked on
sampled rows and columns against the oracle, bit for bit."""
import pytest
import torch

import oracle
from tests._util import assert_bits_equal, encode_dtype, f64, log
import tensor_gemm_collective_amd as tgc

pytestmark = pytest.mark.gpu

LIM = 1 << 31


def _ints(shape, seed, lo=-4, hi=4):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, device="cuda", dtype=torch.int16).to(torch.bfloat16)


def _normal(shape, seed, sigma):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * sigma).to(torch.bfloat16)


def _sample_rows(m, chunks):
    """First and last rows, and both sides of every chunk boundary."""
    rows = {0, 1, m - 2, m - 1}
    for c in range(1, chunks):
        rows |= {c * m // chunks - 1, c * m // chunks}
    return sorted(rows)


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def test_all_reduce_output_just_below_2_31_elements():
    m, n, k, world, rank, split = 32768, 65528, 64, 8, 3, 4
    assert m * n < LIM and m * (n + 8) >= LIM
    log(f"limits: AR bf16 m={m} n={n} k={k} (m*n = {m * n})")
    x, w = _ints((m, k), 1), _ints((k, n), 2)
    peers = [None if r == rank else _normal((m, n), 10 + r, 1.0) for r in range(world)]
    y, p = tgc.matmul_all_reduce(x, w, peers, rank, y=_nan((m, n)), partial_out=_nan((m, n)), split=split,
                                 deterministic=1)
    torch.cuda.synchronize()
    # every element written (outputs started as NaN; the inputs are finite)
    assert bool(torch.isfinite(p).all()) and bool(torch.isfinite(y).all())
    rows = torch.tensor(_sample_rows(m, split), device="cuda")
    xs, ys, ps = f64(x[rows], "bf16"), y[rows], p[rows]
    exact = xs @ f64(w, "bf16")
    assert_bits_equal(ps, encode_dtype(exact, "bf16"), "partial_out rows (integer operands: exact)")
    parts = [f64(ps, "bf16") if r == rank else f64(peers[r][rows], "bf16") for r in range(world)]
    assert_bits_equal(ys, encode_dtype(oracle.reduce_fixed_order(parts, "bf16"), "bf16"), "y rows, fixed order")
    del x, w, peers, y, p
    torch.cuda.empty_cache()


# k = 65472: whole 128-byte rows, so the launch copies the gathered rows itself;
# k = 65528: not a multiple of 32, the matmul with a zero-filled k tail
@pytest.mark.parametrize("k", [65472, 65528])
def test_allgather_gathered_matrix_just_below_2_31_elements(k):
    world, rank, split, n = 8, 6, 4, 64
    shard = 4096
    m = shard * world
    assert m * k < LIM and m * (k + 64) >= LIM
    log(f"limits: AG V2 bf16 m={m} k={k} n={n} (m*k = {m * k})")
    shards = [_ints((shard, k), 20 + r) for r in range(world)]
    w = _ints((k, n), 3, -1, 1)
    peers = [None if r == rank else shards[r] for r in range(world)]
    y, g = tgc.allgather_matmul(shards[rank], peers, w, rank, split=split, v2=True)
    torch.cuda.synchronize()
    rows = _sample_rows(m, world)
    rt = torch.tensor(rows, device="cuda")
    want_g = torch.stack([shards[r // shard][r % shard] for r in rows])
    assert_bits_equal(g[rt], want_g, "gathered rows")
    exact = f64(want_g, "bf16") @ f64(w, "bf16")
    assert_bits_equal(y[rt], encode_dtype(exact, "bf16"), "y rows (integer operands: exact)")
    del shards, w, peers, y, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [65504, 65528])   # the LDS-ring matmul / the zero-filled k tail
def test_weight_just_below_2_31_elements(k):
    m, n, split = 512, 32768, 4
    assert k * n < LIM and (k + 32) * n >= LIM
    log(f"limits: matmul bf16 m={m} n={n} k={k} (k*n = {k * n})")
    x, w = _ints((m, k), 4, -1, 1), _ints((k, n), 5, -1, 1)
    y, p = tgc.matmul_all_reduce(x, w, [None], 0, y=_nan((m, n)), partial_out=_nan((m, n)), split=split,
                                 deterministic=1)
    torch.cuda.synchronize()
    rows = torch.tensor(_sample_rows(m, split), device="cuda")
    cols = torch.tensor(sorted({0, 1, 255, 256, n // 2, n - 2, n - 1}), device="cuda")
    exact = f64(x[rows], "bf16") @ f64(w[:, cols].contiguous(), "bf16")
    assert_bits_equal(p[rows][:, cols].contiguous(), encode_dtype(exact, "bf16"), "partial_out (exact)")
    assert_bits_equal(y, p, "world 1: y == partial_out")
    # every element written (the outputs started as NaN)
    assert bool(torch.isfinite(p).all())
    del x, w, y, p
    torch.cuda.empty_cache()
