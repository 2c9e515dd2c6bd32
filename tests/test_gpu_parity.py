"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle
finishes in seconds (several tiles, ragged tails), plus the properties the
method fixes: bit-exact gather, bitwise-stable deterministic reduction,
chunk-count invariance, reduce-scatter == all-reduce slice.

All calls go through the Python binding into libcoc.so (C ABI).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import (TOL, TORCH_DT, assert_bits_equal, assert_close, dev, encode_dtype, f64,
                         log, raw)

pytestmark = pytest.mark.gpu

WID_TEST = 100   # workload ids >= 100: parity-test inputs


def _ints(tag, shape, lo, hi, dtype):
    return synth.integers(WID_TEST + tag, synth.T_X, 0, shape, lo, hi, dtype)


def _peers_ints(tag, world, rank, shape, dtype, lo=-64, hi=64):
    return [None if r == rank else synth.integers(WID_TEST + tag, synth.T_PEER, r, shape, lo, hi, dtype)
            for r in range(world)]


# ------------------------------------------------------------------ fp32 small case
@pytest.mark.parametrize("split", [1, 2, 4, 8])
@pytest.mark.parametrize("det", [0, 1])
def test_toy_fp32_all_reduce_equals_unsplit_layer(split, det):
    """X 256x512 and W 512x256 uniform[-1,1], K split over tp=2; rank 0 computes
    K shard 0, the peer partial is K shard 1's product (from the oracle)."""
    log(f"toy fp32 AR split={split} det={det}")
    wl = synth.WORKLOADS["toy_f32"]
    xf = synth.uniform(wl.wid, synth.T_X, 0, (256, 512), -1, 1, "f32")
    wf = synth.uniform(wl.wid, synth.T_W, 0, (512, 256), -1, 1, "f32")
    x0, w0 = xf[:, :256].contiguous(), wf[:256].contiguous()
    p1 = oracle.round_f32(oracle.matmul(f64(xf[:, 256:], "f32"), f64(wf[256:], "f32")))
    peer = torch.from_numpy(p1.astype(np.float32))
    y, p = tgc.matmul_all_reduce(dev(x0), dev(w0), [None, dev(peer)], 0, split=split, deterministic=det)
    torch.cuda.synchronize()
    full = oracle.matmul(f64(xf, "f32"), f64(wf, "f32"))
    assert_close(y, full, "f32", "y vs unsplit X_full @ W_full")
    assert_close(p, oracle.matmul(f64(x0, "f32"), f64(w0, "f32")), "f32", "partial_out")


# ------------------------------------------------------------------ exact integer GEMM
GEMM_SHAPES = [
    (300, 200, 136),     # k % 32 != 0: 128x128 kernel with a zero-filled k tail; ragged m, n
    (1, 8, 8),
    (64, 8, 520),
    (517, 1032, 72),
    (2088, 8200, 64),    # ring kernel, 256x256 tiles, ragged m and n
    (1000, 6152, 96),    # ring kernel, 128x256 tiles, ragged m and n
    (300, 1032, 160),    # ring kernel, 128x128 tiles, ragged m and n
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_integer_inputs_bit_exact(dtype, m, n, k):
    """Small integers: the binary32 accumulation is exact, so partial_out must be
    the correctly rounded exact product, bit for bit; y (deterministic) must be
    the fixed-order sum of the stored partials, bit for bit."""
    log(f"integer GEMM {dtype} m={m} n={n} k={k}")
    x = _ints(1, (m, k), -4, 4, dtype)
    w = synth.integers(WID_TEST + 1, synth.T_W, 0, (k, n), -4, 4, dtype)
    peers = _peers_ints(1, 2, 0, (m, n), dtype)
    y, p = tgc.matmul_all_reduce(dev(x), dev(w), [None, dev(peers[1])], 0, split=1, deterministic=1)
    torch.cuda.synchronize()
    exact = oracle.matmul(f64(x, dtype), f64(w, dtype))
    assert_bits_equal(p, encode_dtype(exact, dtype), "partial_out")
    y_ref = oracle.reduce_fixed_order([oracle.round_dtype(exact, dtype), f64(peers[1], dtype)], dtype)
    assert_bits_equal(y, encode_dtype(y_ref, dtype), "y")


def test_gemm_bits_independent_of_kernel_and_tile():
    """Rows 0..127 of X @ W through the 256x256, 128x256 and 128x128 ring tiles
    (k = 512: activations staged two 32-k stages at a time), through the ring
    with single 32-k stages (k padded with zeros to 544, not a multiple of 64)
    and through the any-k kernel (k padded to 520) are the same bits: every
    kernel walks k in the same 16-k MFMA steps, and zero steps add nothing."""
    log("GEMM bits across kernels and tiles")
    k, n = 512, 8192
    x = synth.normal(WID_TEST + 12, synth.T_X, 0, (2048, k), 1.0, "bf16")
    w = synth.normal(WID_TEST + 12, synth.T_W, 0, (k, n), 0.02, "bf16")
    xd, wd = dev(x), dev(w)
    outs = []
    for rows in (2048, 1024, 128):      # 256 tiles of 256x256, 256 of 128x256, 32 of 128x128
        _, p = tgc.matmul_all_reduce(xd[:rows].contiguous(), wd, [None], 0, split=1)
        outs.append(p[:128])
    for pad in (32, 8):
        xpad = torch.zeros((128, k + pad), dtype=torch.bfloat16, device="cuda")
        xpad[:, :k] = xd[:128]
        wpad = torch.zeros((k + pad, n), dtype=torch.bfloat16, device="cuda")
        wpad[:k] = wd
        _, p = tgc.matmul_all_reduce(xpad, wpad, [None], 0, split=1)
        outs.append(p)
    torch.cuda.synchronize()
    for i, o in enumerate(outs[1:], 1):
        assert_bits_equal(o, raw(outs[0]), f"variant {i} vs 256x256 tiles")
    assert_close(outs[0], oracle.matmul(f64(x[:128], "bf16"), f64(w, "bf16")), "bf16", "rows 0..127")


def test_gemm_k_zero_gives_zero_partial():
    log("AR k=0")
    m, n = 64, 64
    x = torch.empty((m, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((0, n), dtype=torch.bfloat16, device="cuda")
    peer = _ints(2, (m, n), -8, 8, "bf16")
    y, p = tgc.matmul_all_reduce(x, w, [None, dev(peer)], 0, split=2, deterministic=1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(p.float()).item() == 0
    assert_bits_equal(y, peer, "y == the peer partial")


# ------------------------------------------------------------------ all-reduce, random values
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_all_reduce_random(dtype, split):
    log(f"AR random {dtype} split={split}")
    m, n, k, world, rank = 512, 1032, 520, 8, 3
    x = synth.normal(WID_TEST + 3, synth.T_X, rank, (m, k), 1.0, dtype)
    w = synth.normal(WID_TEST + 3, synth.T_W, rank, (k, n), 0.02, dtype)
    peers = synth.peers_random(WID_TEST + 3, world, rank, (m, n), 0.46, dtype)
    for det in (0, 1):
        y, p = tgc.matmul_all_reduce(dev(x), dev(w), [dev(q) for q in peers], rank, split=split,
                                     deterministic=det)
        torch.cuda.synchronize()
        y_ref, p_ref = oracle.matmul_all_reduce(f64(x, dtype), f64(w, dtype),
                                                [None if q is None else f64(q, dtype) for q in peers], rank)
        assert_close(p, p_ref, dtype, "partial_out")
        assert_close(y, y_ref, dtype, f"y det={det}")
        if det:
            # deterministic reduction of what is stored, bit for bit
            parts = [f64(p, dtype) if r == rank else f64(peers[r], dtype) for r in range(world)]
            assert_bits_equal(y, encode_dtype(oracle.reduce_fixed_order(parts, dtype), dtype), "y det bits")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("k", [264, 256])
def test_deterministic_bits_independent_of_split_and_run(dtype, k):
    log(f"AR det invariance {dtype} k={k}")
    m, n, world, rank = 256, 512, 8, 6
    x = synth.normal(WID_TEST + 4, synth.T_X, rank, (m, k), 1.0, dtype)
    w = synth.normal(WID_TEST + 4, synth.T_W, rank, (k, n), 0.02, dtype)
    peers = [dev(q) for q in synth.peers_random(WID_TEST + 4, world, rank, (m, n), 0.33, dtype)]
    xd, wd = dev(x), dev(w)
    ref = None
    for split in (1, 2, 4, 8):
        for run in range(10 if split == 4 else 2):
            y, p = tgc.matmul_all_reduce(xd, wd, peers, rank, split=split, deterministic=1)
            torch.cuda.synchronize()
            if ref is None:
                ref = (raw(y), raw(p))
            else:
                assert_bits_equal(y, ref[0], f"y split={split} run={run}")
                assert_bits_equal(p, ref[1], f"partial split={split} run={run}")


# ------------------------------------------------------------------ reduce-scatter
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("split", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [264, 256])
def test_reduce_scatter(dtype, split, k):
    log(f"RS {dtype} split={split} k={k}")
    m, n, world, rank = 1024, 520, 8, 5
    b = m // world
    x = synth.normal(WID_TEST + 5, synth.T_X, rank, (m, k), 1.0, dtype)
    w = synth.normal(WID_TEST + 5, synth.T_W, rank, (k, n), 0.02, dtype)
    peers_full = synth.peers_random(WID_TEST + 5, world, rank, (m, n), 0.33, dtype)
    # only this rank's slice rows of the peers may be read: poison the rest
    peers_rs = []
    for q in peers_full:
        if q is None:
            peers_rs.append(None)
            continue
        z = torch.full((m, n), float("nan"), dtype=TORCH_DT[dtype])
        z[rank * b:(rank + 1) * b] = q[rank * b:(rank + 1) * b]
        peers_rs.append(dev(z))
    xd, wd = dev(x), dev(w)
    for det in (0, 1):
        y, p = tgc.matmul_reduce_scatter(xd, wd, peers_rs, rank, split=split, deterministic=det)
        torch.cuda.synchronize()
        assert y.shape == (b, n)
        y_ref, p_ref = oracle.matmul_reduce_scatter(
            f64(x, dtype), f64(w, dtype), [None if q is None else f64(q, dtype) for q in peers_full], rank)
        assert_close(p, p_ref, dtype, "partial_out")
        assert_close(y, y_ref, dtype, f"y det={det}")
    # deterministic RS == the same rows of deterministic AR, bit for bit
    y_ar, _ = tgc.matmul_all_reduce(xd, wd, [dev(q) for q in peers_full], rank, split=split, deterministic=1)
    y_rs, _ = tgc.matmul_reduce_scatter(xd, wd, peers_rs, rank, split=split, deterministic=1)
    torch.cuda.synchronize()
    assert_bits_equal(y_rs, raw(y_ar)[rank * b:(rank + 1) * b], "RS vs AR slice")


# ------------------------------------------------------------------ all-gather matmul
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("split", [1, 2, 4, 8])
@pytest.mark.parametrize("rank", [0, 5])
@pytest.mark.parametrize("k", [264, 256])
def test_allgather_matmul(dtype, split, rank, k):
    log(f"AG {dtype} split={split} rank={rank} k={k}")
    world, shard, n = 8, 64, 392
    m = world * shard
    shards = [synth.normal(WID_TEST + 6, synth.T_PEER, r, (shard, k), 1.0, dtype) for r in range(world)]
    w = synth.normal(WID_TEST + 6, synth.T_W, 0, (k, n), 0.02, dtype)
    peers = [None if r == rank else dev(shards[r]) for r in range(world)]
    xs, wd = dev(shards[rank]), dev(w)
    y_ref, g_ref = oracle.allgather_matmul([f64(s, dtype) for s in shards], f64(w, dtype))
    y1 = tgc.allgather_matmul(xs, peers, wd, rank, split=split)
    y2, g2 = tgc.allgather_matmul(xs, peers, wd, rank, split=split, v2=True)
    torch.cuda.synchronize()
    assert_bits_equal(g2, torch.cat(shards), "gathered_out (V2)")
    assert_close(y1, y_ref, dtype, "y")
    assert_bits_equal(y2, y1, "V2 y == non-V2 y")
    if split == 1:
        return
    y_s1 = tgc.allgather_matmul(xs, peers, wd, rank, split=1)
    torch.cuda.synchronize()
    assert_bits_equal(y1, y_s1, "y independent of split")


# ------------------------------------------------------------------ backward pair
# dX = dY @ W^T with the forward k x n weight read transposed (trans_w), and
# dW = G^T @ dY (weight_grad).  A transposed operand only changes how the
# tile is staged, so the bits must equal the plain path on the stored
# transpose; the oracle checks the values.
TW_SHAPES = [(528, 392, 256), (2080, 1032, 96), (1024, 8200, 64)]   # m, n (output), k (reduction)


@pytest.mark.parametrize("trans_w", [False, True])
@pytest.mark.parametrize("k", [64, 128, 192, 256, 320, 384])
def test_paired_stage_edges(k, trans_w):
    """k a multiple of 64 stages two 32-k activation stages (and, with transposed
    weights, weight stages) at a time; the schedule has its own code for 2, 4 and
    6 stages and for longer loops.  Integer operands make every sum exact: the
    paired product must be the exact result, and equal bit for bit to the product
    of the same operands padded with 32 zero k (single 32-k stages)."""
    log(f"paired stage edges k={k} trans_w={trans_w}")
    m, n = 512, 768
    x = _ints(20, (m, k), -3, 3, "bf16")
    w = synth.integers(WID_TEST + 20, synth.T_W, 0, (k, n), -3, 3, "bf16")
    exact = oracle.matmul(f64(x, "bf16"), f64(w, "bf16"))
    outs = []
    for pad in (0, 32):
        xp = torch.zeros((m, k + pad), dtype=torch.bfloat16)
        xp[:, :k] = x
        wp = torch.zeros((k + pad, n), dtype=torch.bfloat16)
        wp[:k] = w
        wd = dev(wp.t().contiguous()) if trans_w else dev(wp)
        _, p = tgc.matmul_all_reduce(dev(xp), wd, [None], 0, split=4, deterministic=1, trans_w=trans_w)
        torch.cuda.synchronize()
        outs.append(p)
    assert_bits_equal(outs[0], encode_dtype(exact, "bf16"), "paired stages vs the exact product")
    assert_bits_equal(outs[1], raw(outs[0]), "single 32-k stages vs paired")


def _nt_operands(kind, m, n, k, dtype, seed):
    """Activations m x k and transposed weights n x k: N(0,1) x N(0,0.02^2);
    'wide': both scaled by powers of two per row, over 2^-12 .. 2^12 (bf16) or
    2^-3 .. 2^3 (fp16, whose outputs must stay below 65504); 'cancel':
    the second half of k repeats the first with the activations negated and
    perturbed by one part in 2^7, so each output is a small difference of
    large partial sums (its rounding depends on the order of the adds)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(m, k, generator=g, dtype=torch.float64)
    w = torch.randn(n, k, generator=g, dtype=torch.float64) * 0.02
    if kind == "wide":
        e = 12 if dtype == "bf16" else 3
        x = x * torch.pow(2.0, torch.randint(-e, e + 1, (m, 1), generator=g).double())
        w = w * torch.pow(2.0, torch.randint(-e, e + 1, (n, 1), generator=g).double())
    elif kind == "cancel":
        h = k // 2
        x[:, h:] = -x[:, :h] * (1 + torch.randn(m, h, generator=g, dtype=torch.float64) / 128)
        w[:, h:] = w[:, :h]
    return x.to(TORCH_DT[dtype]), w.to(TORCH_DT[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kind", ["normal", "wide", "cancel"])
@pytest.mark.parametrize("m,n,k", [(4096, 4096, 64), (4096, 4096, 128), (4096, 4096, 192), (4000, 4104, 320),
                                   (4096, 4352, 1024)])
def test_four_wave_tile_same_bits(dtype, kind, m, n, k, monkeypatch):
    """A lone matmul with transposed weights and 256 x 256 tiles (k % 64 ==
    0) runs the four-wave tile (four 128 x 128 waves of 16x16x32 MFMAs);
    COC_FOUR_WAVE=0 makes the same launch run the eight-wave ring tile
    (32x32x16 MFMAs).  Both add each output's products in the same 8-k steps
    in increasing k, so the partials must be the same bits, also on operands
    whose sums cancel or span a wide exponent range, and on ragged m and n;
    k = 64, 128 and 192 take the schedule's one-, two- and three-stage paths."""
    log(f"four-wave vs eight-wave tile {dtype} {kind} m={m} n={n} k={k}")
    x, wt = _nt_operands(kind, m, n, k, dtype, 7 + m + n + k)
    xd, wtd = dev(x), dev(wt)
    outs = {}
    for v in ("1", "0"):
        monkeypatch.setenv("COC_FOUR_WAVE", v)
        _, p = tgc.matmul_all_reduce(xd, wtd, [None], 0, split=1, trans_w=True)
        torch.cuda.synchronize()
        outs[v] = p
    monkeypatch.delenv("COC_FOUR_WAVE")
    assert torch.isfinite(outs["1"].float()).all()
    assert_bits_equal(outs["1"], raw(outs["0"]), "four-wave vs eight-wave tile")
    if kind == "normal":
        rows = torch.arange(0, m, 97)
        want = oracle.matmul(f64(x[rows], dtype), f64(wt, dtype).T)
        assert_close(outs["1"][rows.to(outs["1"].device)], want, dtype, "sampled rows vs the oracle")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", TW_SHAPES)
@pytest.mark.parametrize("split", [1, 4])
def test_transposed_weights_compute_first(dtype, m, n, k, split):
    log(f"trans_w AR/RS {dtype} m={m} n={n} k={k} split={split}")
    world, rank = 4, 1
    x = synth.normal(WID_TEST + 31, synth.T_X, rank, (m, k), 1.0, dtype)
    w = synth.normal(WID_TEST + 31, synth.T_W, rank, (k, n), 0.02, dtype)   # the product's k x n weight
    peers = synth.peers_random(WID_TEST + 31, world, rank, (m, n), 0.3, dtype)
    xd, wd, wtd = dev(x), dev(w), dev(w).t().contiguous()                   # wtd: n x k, as stored
    pd = [dev(q) for q in peers]
    y_t, p_t = tgc.matmul_all_reduce(xd, wtd, pd, rank, split=split, deterministic=1, trans_w=True)
    y_n, p_n = tgc.matmul_all_reduce(xd, wd, pd, rank, split=split, deterministic=1)
    r_t, _ = tgc.matmul_reduce_scatter(xd, wtd, pd, rank, split=split, deterministic=1, trans_w=True)
    r_n, _ = tgc.matmul_reduce_scatter(xd, wd, pd, rank, split=split, deterministic=1)
    torch.cuda.synchronize()
    assert_bits_equal(p_t, p_n, "partial_out, transposed weights")
    assert_bits_equal(y_t, y_n, "all-reduce, transposed weights")
    assert_bits_equal(r_t, r_n, "reduce-scatter, transposed weights")
    y_ref, p_ref = oracle.matmul_all_reduce(f64(x, dtype), f64(w, dtype),
                                            [None if q is None else f64(q, dtype) for q in peers], rank)
    assert_close(p_t, p_ref, dtype, "partial_out")
    assert_close(y_t, y_ref, dtype, "y")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("split", [1, 4, 8])
@pytest.mark.parametrize("rank", [0, 5])
def test_transposed_weights_allgather(dtype, split, rank):
    log(f"trans_w AG {dtype} split={split} rank={rank}")
    world, shard, n, k = 8, 64, 392, 256
    shards = [synth.normal(WID_TEST + 32, synth.T_PEER, r, (shard, k), 1.0, dtype) for r in range(world)]
    w = synth.normal(WID_TEST + 32, synth.T_W, 0, (k, n), 0.02, dtype)
    peers = [None if r == rank else dev(shards[r]) for r in range(world)]
    xs, wd = dev(shards[rank]), dev(w)
    y_t, g_t = tgc.allgather_matmul(xs, peers, wd.t().contiguous(), rank, split=split, v2=True, trans_w=True)
    y_n = tgc.allgather_matmul(xs, peers, wd, rank, split=split)
    torch.cuda.synchronize()
    assert_bits_equal(g_t, torch.cat(shards), "gathered_out")
    assert_bits_equal(y_t, y_n, "all-gather matmul, transposed weights")
    y_ref, _ = oracle.allgather_matmul([f64(s, dtype) for s in shards], f64(w, dtype))
    assert_close(y_t, y_ref, dtype, "y")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("m,k,n", [(64, 520, 1040), (2048, 264, 392), (96, 1032, 8200), (4096, 256, 512)])
def test_weight_grad(dtype, m, k, n):
    log(f"weight_grad {dtype} m={m} k={k} n={n}")
    g = synth.normal(WID_TEST + 33, synth.T_X, 0, (m, k), 1.0, dtype)
    dy = synth.normal(WID_TEST + 33, synth.T_W, 0, (m, n), 1.0, dtype)
    gd, dyd = dev(g), dev(dy)
    dw = tgc.weight_grad(gd, dyd)
    # the plain matmul on G^T as stored (world 1: partial_out = G^T @ dY)
    _, p = tgc.matmul_all_reduce(gd.t().contiguous(), dyd, [None], 0, split=1)
    torch.cuda.synchronize()
    assert dw.shape == (k, n)
    assert_bits_equal(dw, p, "weight_grad vs the plain matmul on G^T")
    assert_close(dw, oracle.weight_grad(f64(g, dtype), f64(dy, dtype)), dtype, "dW")


def test_weight_grad_of_gathered_matrix():
    """The backward of the sequence-parallel pair at small scale: V2's gathered
    G reused for dW, and dX = AG(dY) @ W^T through the all-gather op."""
    world, shard, k, n, rank = 4, 64, 264, 384, 2   # n: the reduction of dX, a multiple of 32
    dt = "bf16"
    shards = [synth.normal(WID_TEST + 34, synth.T_PEER, r, (shard, k), 1.0, dt) for r in range(world)]
    w = synth.normal(WID_TEST + 34, synth.T_W, 0, (k, n), 0.02, dt)
    dys = [synth.normal(WID_TEST + 34, synth.T_X, r, (shard, n), 1.0, dt) for r in range(world)]
    peers = [None if r == rank else dev(shards[r]) for r in range(world)]
    _, g = tgc.allgather_matmul(dev(shards[rank]), peers, dev(w), rank, split=4, v2=True)
    dy_full = dev(torch.cat(dys))
    dw = tgc.weight_grad(g, dy_full)
    dpeers = [None if r == rank else dev(dys[r]) for r in range(world)]
    dx = tgc.allgather_matmul(dev(dys[rank]), dpeers, dev(w), rank, split=4, trans_w=True)   # (m x n) @ W^T
    torch.cuda.synchronize()
    G = oracle.allgather([f64(s, dt) for s in shards])
    DY = oracle.allgather([f64(d, dt) for d in dys])
    assert_close(dw, oracle.weight_grad(G, DY), dt, "dW")
    assert_close(dx, oracle.matmul(DY, f64(w, dt).T), dt, "dX")


# ------------------------------------------------------------------ w8a16
# a per-group scale table needs the group to divide k
_W8_EXACT = [(mode, split, n, g, k) for k in (512, 544) for n, g in ((520, 128), (1040, 128), (1040, 32), (528, 16))
             for split in (1, 4) for mode in ("per_tensor", "per_channel", "per_group")
             if not (mode == "per_group" and k % g)]


@pytest.mark.parametrize("mode,split,n,g,k", _W8_EXACT)
def test_w8a16_exact_with_power_of_two_scales(mode, split, n, g, k):
    """X in {-2..2}, q in {-15..15}, scales 2^-6..2^-2 differing per channel and
    group: every product and the binary32 sums are exact, so partial_out is the
    correctly rounded exact result, bit for bit, whatever the scale index.
    n % 16 == 0 with group a multiple of 32 takes the ring kernel (int8
    transpose reads, in-register dequantisation; k = 512 stages the
    activations two 32-k stages at a time, k = 544 one); the others the
    register-staged kernel."""
    log(f"w8a16 exact {mode} split={split} n={n} g={g} k={k}")
    m, world, rank = 256, 4, 1
    x = _ints(7, (m, k), -2, 2, "f16")
    q = synth.integers(WID_TEST + 7, synth.T_W, 0, (k, n), -15, 15, "i8")
    shape = {"per_tensor": (1,), "per_channel": (n,), "per_group": (k // g, n)}[mode]
    s = synth.pow2_scales(WID_TEST + 7, 0, shape)
    peers = _peers_ints(7, world, rank, (m, n), "f16")
    y, p = tgc.matmul_all_reduce_w8a16(dev(x), dev(q), dev(s), mode, [dev(t) for t in peers], rank,
                                       group_size=g, split=split, deterministic=1)
    torch.cuda.synchronize()
    exact = oracle.matmul(f64(x, "f16"), oracle.dequant_weight(q.numpy(), f64(s, "f16"), mode, g))
    assert_bits_equal(p, encode_dtype(exact, "f16"), "partial_out")
    parts = [oracle.round_dtype(exact, "f16") if r == rank else f64(peers[r], "f16") for r in range(world)]
    assert_bits_equal(y, encode_dtype(oracle.reduce_fixed_order(parts, "f16"), "f16"), "y")


@pytest.mark.parametrize("mode,group", [("per_tensor", 0), ("per_channel", 0), ("per_group", 128),
                                        ("per_group", 64), ("per_group", 16)])
def test_w8a16_random(mode, group):
    log(f"w8a16 random {mode} g={group}")
    m, n, k, world, rank = 384, 1024, 512, 8, 2
    x = synth.normal(WID_TEST + 8, synth.T_X, 0, (m, k), 1.0, "f16")
    q = synth.integers(WID_TEST + 8, synth.T_W, 0, (k, n), -127, 127, "i8")
    shape = {"per_tensor": (1,), "per_channel": (n,), "per_group": (k // max(group, 1), n)}[mode]
    s = synth.fp16_scales(WID_TEST + 8, 0, shape)
    peers = synth.peers_random(WID_TEST + 8, world, rank, (m, n), 20.0, "f16")
    y, p = tgc.matmul_all_reduce_w8a16(dev(x), dev(q), dev(s), mode, [dev(t) for t in peers], rank,
                                       group_size=group, split=4, deterministic=0)
    torch.cuda.synchronize()
    y_ref, p_ref = oracle.matmul_all_reduce_w8a16(
        f64(x, "f16"), q.numpy(), f64(s, "f16"), mode, group,
        [None if t is None else f64(t, "f16") for t in peers], rank)
    assert_close(p, p_ref, "f16", "partial_out")
    assert_close(y, y_ref, "f16", "y")


# ------------------------------------------------------------------ edge cases and semantics
def test_world_one_is_plain_matmul():
    log("AR world=1")
    x = synth.normal(WID_TEST + 9, synth.T_X, 0, (128, 64), 1.0, "bf16")
    w = synth.normal(WID_TEST + 9, synth.T_W, 0, (64, 96), 0.02, "bf16")
    y, p = tgc.matmul_all_reduce(dev(x), dev(w), [None], 0, split=4, deterministic=1)
    torch.cuda.synchronize()
    assert_bits_equal(y, p, "y == partial_out")
    assert_close(p, oracle.matmul(f64(x, "bf16"), f64(w, "bf16")), "bf16", "partial_out")


def test_empty_m_is_noop():
    log("AR m=0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    y, p = tgc.matmul_all_reduce(x, w, [None, torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")], 0)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


def test_outputs_guard_bands_untouched():
    """Outputs placed inside larger buffers: nothing outside them is written."""
    log("AR guard bands")
    m, n, k, world = 256, 264, 128, 4
    x = synth.normal(WID_TEST + 10, synth.T_X, 0, (m, k), 1.0, "bf16")
    w = synth.normal(WID_TEST + 10, synth.T_W, 0, (k, n), 0.02, "bf16")
    peers = [dev(q) for q in synth.peers_random(WID_TEST + 10, world, 0, (m, n), 0.2, "bf16")]
    pad = 64 * n      # 64 rows of guard on each side (16-byte aligned offsets)
    ybuf = torch.full((m * n + 2 * pad,), 12345.0, dtype=torch.bfloat16, device="cuda")
    pbuf = torch.full((m * n + 2 * pad,), -777.0, dtype=torch.bfloat16, device="cuda")
    y = ybuf[pad:pad + m * n].view(m, n)
    p = pbuf[pad:pad + m * n].view(m, n)
    tgc.matmul_all_reduce(dev(x), dev(w), peers, 0, y=y, partial_out=p, split=4, deterministic=1)
    torch.cuda.synchronize()
    for buf, val in ((ybuf, 12345.0), (pbuf, -777.0)):
        assert torch.all(buf[:pad] == val) and torch.all(buf[pad + m * n:] == val)
    assert_close(p, oracle.matmul(f64(x, "bf16"), f64(w, "bf16")), "bf16", "partial_out")


def test_invalid_arguments_enqueue_nothing():
    log("AR error paths with real tensors")
    m, n, k = 64, 64, 64
    x = torch.ones((m + 1, k), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((k, n), dtype=torch.bfloat16, device="cuda")
    peers = [None, torch.ones((m, n), dtype=torch.bfloat16, device="cuda")]
    y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda")
    p = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda")
    # misaligned x (one element into the buffer)
    xv = x.view(-1)[1:1 + m * k].view(m, k)
    with pytest.raises(tgc.CocError) as ei:
        tgc.matmul_all_reduce(xv, w, peers, 0, y=y, partial_out=p)
    assert ei.value.status_name == "COC_ERR_ALIGN"
    with pytest.raises(tgc.CocError) as ei:
        tgc.matmul_all_reduce(x[:m], w, peers, 0, y=y, partial_out=p, split=3)
    assert ei.value.status_name == "COC_ERR_SPLIT"
    with pytest.raises(tgc.CocError) as ei:
        tgc.matmul_all_reduce(x[:m], w, peers, 0, y=y, partial_out=y)
    assert ei.value.status_name == "COC_ERR_ALIAS"
    torch.cuda.synchronize()
    assert torch.all(y == 3.0) and torch.all(p == 3.0)


def test_stream_order_without_host_sync():
    """Outputs are visible to later work on the caller's stream with no host sync."""
    log("stream semantics")
    m, n, k, world = 512, 512, 256, 8
    x = dev(synth.normal(WID_TEST + 11, synth.T_X, 0, (m, k), 1.0, "bf16"))
    w = dev(synth.normal(WID_TEST + 11, synth.T_W, 0, (k, n), 0.02, "bf16"))
    peers = [dev(q) for q in synth.peers_random(WID_TEST + 11, world, 0, (m, n), 0.3, "bf16")]
    y_ref, _ = tgc.matmul_all_reduce(x, w, peers, 0, split=4, deterministic=1)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = []
        for _ in range(4):
            y, _ = tgc.matmul_all_reduce(x, w, peers, 0, split=4, deterministic=1)
            outs.append(y.clone())       # consumer on the same stream, no sync
            y.fill_(0)
    s.synchronize()
    for o in outs:
        assert_bits_equal(o, y_ref, "consumer on caller stream")


# ------------------------------------------------------------------ one-launch pipeline hand-over
@pytest.mark.parametrize("world,rank,dt", [(8, 0, "bf16"), (8, 5, "bf16"), (4, 3, "bf16"), (8, 7, "f16")])
def test_allgather_fused_copy_handover(world, rank, dt):
    """The all-gather shape where the matmul launch copies the rows itself
    (448 tiles of 256 x 256 on 256 workgroups: some own a single tile).  Two
    input sets alternate through the same buffers over every split, so rows
    read before their copy landed, or counters left out of step by an
    earlier call, would show: each call must match split 1 bit for bit."""
    k, n = 256, 7168
    m = 4096
    shard = m // world
    sets = []
    for tag in (21, 22):
        shards = [synth.normal(WID_TEST + tag, synth.T_PEER, r, (shard, k), 1.0, dt) for r in range(world)]
        sets.append([dev(s) for s in shards])
    w = dev(synth.normal(WID_TEST + 21, synth.T_W, 0, (k, n), 0.02, dt))
    peers_of = lambda sh: [None if r == rank else sh[r] for r in range(world)]
    refs = [tgc.allgather_matmul(sh[rank], peers_of(sh), w, rank, split=1) for sh in sets]
    torch.cuda.synchronize()
    y = torch.empty((m, n), dtype=TORCH_DT[dt], device="cuda")
    g = torch.empty((m, k), dtype=TORCH_DT[dt], device="cuda")
    for it, split in enumerate((4, 8, 2, 4, 8, 2)):
        sh = sets[it % 2]
        log(f"fused all-gather copy, world={world} rank={rank} {dt} call {it} split={split}")
        tgc.allgather_matmul(sh[rank], peers_of(sh), w, rank, y=y, gathered_out=g, v2=True, split=split)
        torch.cuda.synchronize()
        assert_bits_equal(g, torch.cat(sh), f"gathered rows, call {it}")
        assert_bits_equal(y, refs[it % 2], f"all-gather matmul, call {it} split {split}")


def test_bounded_wait_gives_up_to_nan(monkeypatch):
    """A hand-over wait whose count never arrives gives up after its poll limit
    (forced from the host: a tiny limit and targets out of reach) and writes
    NaN where it would have read unready data; every kernel ends, the call
    succeeds, what needed no wait is exact, and the next normal call is exact
    again (the counter bookkeeping stayed in step)."""
    bf = torch.bfloat16
    g0 = torch.Generator(device="cuda").manual_seed(5)
    # all-gather matmul whose launch copies the rows itself (rank 0: own rows 0..511)
    world, shard, k, n, rank = 8, 512, 256, 7168, 0
    shards = [torch.randn(shard, k, device="cuda", generator=g0).to(bf) for _ in range(world)]
    w = (torch.randn(k, n, device="cuda", generator=g0) * 0.02).to(bf)
    peers = [None if r == rank else shards[r] for r in range(world)]
    ref = tgc.allgather_matmul(shards[rank], peers, w, rank, split=1)
    # reduce-scatter whose first two chunks reduce beside the matmul (512 tiles, two rounds)
    m2, n2, k2, rank2 = 4096, 8192, 256, 3
    x2 = torch.randn(m2, k2, device="cuda", generator=g0).to(bf)
    w2 = (torch.randn(k2, n2, device="cuda", generator=g0) * 0.02).to(bf)
    peers2 = [None if r == rank2 else torch.randn(m2, n2, device="cuda", generator=g0).to(bf) for r in range(world)]
    ref2, _ = tgc.matmul_reduce_scatter(x2, w2, peers2, rank2, split=1, deterministic=1)
    torch.cuda.synchronize()

    log("hand-over waits forced to give up (COC_SPIN_LIMIT=64, unreachable targets)")
    monkeypatch.setenv("COC_SPIN_LIMIT", "64")
    monkeypatch.setenv("COC_TEST_UNREACHABLE_WAIT", "1")
    y, g = tgc.allgather_matmul(shards[rank], peers, w, rank, split=4, v2=True)
    y2, p2 = tgc.matmul_reduce_scatter(x2, w2, peers2, rank2, split=4, deterministic=1)
    torch.cuda.synchronize()
    assert_bits_equal(g, torch.cat(shards), "the copy itself still completes")
    assert_bits_equal(y[:shard], ref[:shard], "own-shard rows (no wait)")
    assert torch.isnan(y[shard:].float()).all(), "rows whose wait gave up must be NaN"
    q = m2 // world // 4   # rows of each chunk in this rank's slice
    assert torch.isnan(y2[:2 * q].float()).all(), "chunks reduced beside the matmul must be NaN"
    assert_bits_equal(y2[2 * q:], ref2[2 * q:], "chunks reduced after the matmul (no wait)")
    assert torch.isfinite(p2.float()).all()
    # the host sees the time-out, once: the check clears the record
    with pytest.raises(tgc.CocError) as ei:
        tgc.check_waits()
    assert ei.value.status_name == "COC_ERR_TIMEOUT"
    tgc.check_waits()

    monkeypatch.delenv("COC_SPIN_LIMIT")
    monkeypatch.delenv("COC_TEST_UNREACHABLE_WAIT")
    log("the next normal calls")
    y, g = tgc.allgather_matmul(shards[rank], peers, w, rank, split=4, v2=True)
    y2, _ = tgc.matmul_reduce_scatter(x2, w2, peers2, rank2, split=4, deterministic=1)
    torch.cuda.synchronize()
    assert_bits_equal(y, ref, "all-gather matmul after the forced time-out")
    assert_bits_equal(y2, ref2, "reduce-scatter after the forced time-out")
    tgc.check_waits()   # no wait gave up this time


def test_waiting_calls_from_two_streams_at_once():
    """Two host threads, each on a stream of its own, issue the one-launch
    pipelines at the same time: the all-gather matmul whose launch copies the
    rows itself (its workgroups wait on one another) and the reduce-scatter
    whose early chunks reduce beside the matmul (the reduce waits on it).  The
    library keeps such calls from running at once on the device, so none of
    their waits can run out for lack of room: every result matches the serial
    form (split 1) bit for bit."""
    import threading
    bf = torch.bfloat16
    g0 = torch.Generator(device="cuda").manual_seed(9)
    world, shard, k, n, rank = 8, 512, 256, 7168, 5
    shards = [torch.randn(shard, k, device="cuda", generator=g0).to(bf) for _ in range(world)]
    w = (torch.randn(k, n, device="cuda", generator=g0) * 0.02).to(bf)
    peers = [None if r == rank else shards[r] for r in range(world)]
    m2, n2, k2, rank2 = 4096, 8192, 256, 3
    x2 = torch.randn(m2, k2, device="cuda", generator=g0).to(bf)
    w2 = (torch.randn(k2, n2, device="cuda", generator=g0) * 0.02).to(bf)
    peers2 = [None if r == rank2 else torch.randn(m2, n2, device="cuda", generator=g0).to(bf) for r in range(world)]
    ref = tgc.allgather_matmul(shards[rank], peers, w, rank, split=1)
    ref2, _ = tgc.matmul_reduce_scatter(x2, w2, peers2, rank2, split=1, deterministic=1)
    torch.cuda.synchronize()

    calls = 6
    outs = [[None] * calls for _ in range(2)]
    errors = []
    start = threading.Barrier(2)

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                for i in range(calls):
                    if (i + t) % 2 == 0:
                        outs[t][i] = tgc.allgather_matmul(shards[rank], peers, w, rank, split=4, v2=True)[0]
                    else:
                        outs[t][i] = tgc.matmul_reduce_scatter(x2, w2, peers2, rank2, split=4,
                                                               deterministic=1)[0]
            s.synchronize()
        except Exception as e:   # reported on the main thread
            errors.append(e)

    log("one-launch pipelines from two threads / two streams at once")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(2):
        for i in range(calls):
            want = ref if (i + t) % 2 == 0 else ref2
            assert_bits_equal(outs[t][i], want, f"thread {t} call {i}")


@pytest.mark.parametrize("split", [2, 4, 8])
def test_pipeline_handover_reuses_buffers_without_stale_rows(split):
    """Two input sets alternate through the same output / gathered buffers, so
    any row the matmul read or the reduce saw from the previous call would show
    up.  Results must match split 1 (one serial matmul, no hand-over) bit for
    bit, and the gathered rows the shards exactly."""
    log(f"pipeline hand-over, split={split}")
    world, rank, shard, k, n = 8, 2, 512, 1024, 2048
    m = world * shard
    sets = []
    for tag in (13, 14):
        shards = [synth.normal(WID_TEST + tag, synth.T_PEER, r, (shard, k), 1.0, "bf16") for r in range(world)]
        x = synth.normal(WID_TEST + tag, synth.T_X, rank, (m, k), 1.0, "bf16")
        peers = synth.peers_random(WID_TEST + tag, world, rank, (m, n), 0.3, "bf16")
        sets.append(([dev(s) for s in shards], dev(x), [dev(q) for q in peers]))
    w = dev(synth.normal(WID_TEST + 13, synth.T_W, 0, (k, n), 0.02, "bf16"))
    refs = []
    for shards, x, peers in sets:
        ag = tgc.allgather_matmul(shards[rank], [None if r == rank else shards[r] for r in range(world)], w, rank,
                                  split=1)
        ar, part = tgc.matmul_all_reduce(x, w, peers, rank, split=1, deterministic=1)
        refs.append((ag, ar, part))
    torch.cuda.synchronize()
    y_ag = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((m, k), dtype=torch.bfloat16, device="cuda")
    y_ar = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    p_ar = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    for it in range(4):
        shards, x, peers = sets[it % 2]
        ref_ag, ref_ar, ref_p = refs[it % 2]
        tgc.allgather_matmul(shards[rank], [None if r == rank else shards[r] for r in range(world)], w, rank,
                             y=y_ag, gathered_out=g, v2=True, split=split)
        tgc.matmul_all_reduce(x, w, peers, rank, y=y_ar, partial_out=p_ar, split=split, deterministic=1)
        torch.cuda.synchronize()
        assert_bits_equal(g, torch.cat(shards), f"gathered rows, call {it}")
        assert_bits_equal(y_ag, ref_ag, f"all-gather matmul, call {it}")
        assert_bits_equal(p_ar, ref_p, f"partial, call {it}")
        assert_bits_equal(y_ar, ref_ar, f"all-reduce, call {it}")


def test_activity_stamps_change_nothing_and_stay_in_bounds():
    """The kernels' activity records (a measurement hook): with them on, every
    output keeps its bits; the records name the launches' kinds with start <=
    end, inside the slots handed out; a buffer too small for a launch gets no
    records from it and nothing past it is written."""
    bf = torch.bfloat16
    g0 = torch.Generator(device="cuda").manual_seed(21)
    world, rank, m, n, k = 8, 2, 4096, 8192, 256
    x = torch.randn(m, k, device="cuda", generator=g0).to(bf)
    w = (torch.randn(k, n, device="cuda", generator=g0) * 0.02).to(bf)
    peers = [None if r == rank else torch.randn(m // world, n, device="cuda", generator=g0).to(bf)
             for r in range(world)]
    full = [None if p is None else torch.cat([p] * world) for p in peers]
    shards = [torch.randn(512, k, device="cuda", generator=g0).to(bf) for _ in range(world)]
    speers = [None if r == rank else shards[r] for r in range(world)]
    want_rs, want_p = tgc.matmul_reduce_scatter(x, w, full, rank, split=4, deterministic=1)
    want_ag = tgc.allgather_matmul(shards[rank], speers, w, rank, split=4)
    torch.cuda.synchronize()
    for cap in (1 << 14, 3):
        log(f"activity stamps, capacity {cap}")
        whole = torch.full((3 * cap + 64,), -7, dtype=torch.int64, device="cuda")
        buf = whole[:3 * cap]
        buf.zero_()
        torch.cuda.synchronize()
        tgc.profile_stamps(buf)
        try:
            y, p = tgc.matmul_reduce_scatter(x, w, full, rank, split=4, deterministic=1)
            ya = tgc.allgather_matmul(shards[rank], speers, w, rank, split=4)
            torch.cuda.synchronize()
            used = tgc.profile_stamp_count()
        finally:
            tgc.profile_stamps(None)
        assert_bits_equal(y, want_rs, "reduce-scatter with stamps")
        assert_bits_equal(p, want_p, "partial with stamps")
        assert_bits_equal(ya, want_ag, "all-gather matmul with stamps")
        h = whole.cpu().numpy()
        assert (h[3 * cap:] == -7).all(), "a record was written past the buffer"
        assert 0 <= used <= cap
        recs = h[:3 * cap].reshape(cap, 3)
        assert not recs[used:].any(), "a record was written outside the slots handed out"
        written = recs[:used][recs[:used, 0] != 0]
        kinds = set((int(v) & 255) - 1 for v in written[:, 0])
        assert kinds <= {0, 1, 2}
        assert (written[:, 1] <= written[:, 2]).all() and (written[:, 1] > 0).all()
        if cap > 3:
            assert kinds == {0, 1, 2}, kinds
        else:
            assert used == 0 and len(written) == 0


@pytest.mark.gpu
def test_mfma_loop_diagnostic_sums_exactly():
    """coc_diag_mfma_loop with every operand 1.0: each of a thread's 8 x 16
    accumulator elements gains 16 per iteration, so each output is 2048 x iters
    exactly (bf16 products of ones, binary32 sums of small integers)."""
    import torch
    log("mfma loop diagnostic, 3 workgroups, 5 iterations")
    ops = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    out = torch.full((3 * 256,), -1.0, dtype=torch.float32, device="cuda")
    flops = tgc.diag_mfma_loop(ops, out, 3, 5)
    torch.cuda.synchronize()
    assert flops == 3 * 4 * 5 * 8 * 32768
    assert torch.equal(out, torch.full_like(out, 2048.0 * 5))
