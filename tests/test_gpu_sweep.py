"""Seeded sweep over shapes and options of every op, against the oracle
(the matmul-collective ops here; the MoE pair and the weight gradient below).

Each case draws, from its own seed: the op (all-reduce, reduce-scatter,
all-gather, all-gather V2, w8A16 all-reduce), the dtype, world size and rank,
split, the deterministic flag, transposed weights, and m, n, k within the
boundary's rules (n, k multiples of 8, k of 32 with transposed weights; m a
multiple of what the op's chunking needs).  The sizes span the tile-shape choices (256 x 256, 128 x 256,
128 x 128), k with and without a 32-multiple (the ring and the zero-filled
k-tail kernels), int8 weights with n a multiple of 16 or not (ring or
register-staged kernel) and every scale mode.

Half the cases use small integers: every binary32 sum is then exact, so the
partial product must equal the correctly rounded exact product bit for bit,
the gathered matrix the shards' bits, and a deterministic output the
fixed-order sum of the stored partials (CoC guide, fused-operator list: the
deterministic variants).  The other half use normally distributed values,
compared normwise at the dtype's tolerance.

All calls go through the Python binding into libcoc.so (C ABI).
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import assert_bits_equal, assert_close, dev, encode_dtype, f64, log, raw

pytestmark = pytest.mark.gpu

WID_SWEEP = 400   # workload ids >= 400: sweep inputs (one per case)
N_CASES = 160


def _draw(i):
    r = random.Random(7919 * (i + 1))
    op = r.choice(["ar", "rs", "ag", "ag_v2", "w8"])
    dt = "f16" if op == "w8" else r.choice(["bf16", "f16"])
    world = r.choice([1, 2, 4, 8])
    rank = r.randrange(world)
    split = r.choice([1, 2, 4, 8])
    det = r.randrange(2)
    trans_w = op != "w8" and r.random() < 0.3
    if op in ("ar", "w8"):
        unit = split
    elif op == "rs":
        unit = world * split
    else:
        unit = world * split // math.gcd(world, split)
    # sizes: mostly up to ~2k rows / columns, sometimes a single tile or less
    m = unit * r.randint(1, max(1, (r.choice([64, 2100, 2100]) // unit)))
    # n and k: multiples of 8, half of n and most of k also of 16 / 32 (the
    # int8 ring kernel and the bf16 / fp16 ring kernels)
    nq = 16 if r.random() < 0.5 else 8
    n = nq * r.randint(1, r.choice([4, 2080 // nq, 2080 // nq]))
    kq = 32 if r.random() < 0.6 or trans_w else 8   # transposed weights need k % 32 == 0
    k = kq * r.randint(1, r.choice([4, 1056 // kq, 1056 // kq]))
    integer = r.random() < 0.5
    mode, group = None, 0
    if op == "w8":
        mode = r.choice(["per_tensor", "per_channel", "per_group"])
        if mode == "per_group":
            group = r.choice([g for g in (8, 16, 32, 64, 128, 256) if k % g == 0])
    return dict(i=i, op=op, dt=dt, world=world, rank=rank, split=split, det=det, trans_w=trans_w,
                m=m, n=n, k=k, integer=integer, mode=mode, group=group)


CASES = [_draw(i) for i in range(N_CASES)]


def _id(c):
    extra = f"-{c['mode']}{c['group'] or ''}" if c["op"] == "w8" else ""
    return (f"{c['i']:02d}-{c['op']}-{c['dt']}-w{c['world']}r{c['rank']}-s{c['split']}-d{c['det']}"
            f"-t{int(c['trans_w'])}-{c['m']}x{c['n']}x{c['k']}-{'int' if c['integer'] else 'rnd'}{extra}")


def _values(c, tensor, idx, shape, dtype, lo, hi, sigma):
    wid = WID_SWEEP + c["i"]
    if c["integer"]:
        return synth.integers(wid, tensor, idx, shape, lo, hi, dtype)
    return synth.normal(wid, tensor, idx, shape, sigma, dtype)


def _weight(c):
    """The weight as stored (k x n, or n x k when trans_w) and its k x n float64 value."""
    k, n, dt = c["k"], c["n"], c["dt"]
    shape = (n, k) if c["trans_w"] else (k, n)
    w = _values(c, synth.T_W, 0, shape, dt, -4, 4, 0.05)
    w64 = f64(w, dt)
    return w, (w64.T if c["trans_w"] else w64)


def _peer_sigma(c):
    return 0.05 * math.sqrt(c["k"])


def _check_reduce(c, y, p, p_exact, peers, rows, what):
    """y against the reduction of the stored partial and the peers over `rows`:
    bit for bit in the fixed order when deterministic with integer inputs,
    normwise otherwise.  p_exact: float64 partial product."""
    dt, rank = c["dt"], c["rank"]
    if c["integer"]:
        assert_bits_equal(p, encode_dtype(p_exact, dt), f"{what} partial_out")
    else:
        assert_close(p, p_exact, dt, f"{what} partial_out")
    own = f64(p, dt)[rows]
    parts = [own if r == rank else f64(peers[r], dt)[rows] for r in range(c["world"])]
    if c["det"] and c["integer"]:
        assert_bits_equal(y, encode_dtype(oracle.reduce_fixed_order(parts, dt), dt), f"{what} y (fixed order)")
    ref = p_exact[rows] + sum(f64(peers[r], dt)[rows] for r in range(c["world"]) if r != rank)
    assert_close(y, ref, dt, f"{what} y")


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_sweep(c):
    log(f"sweep {_id(c)}")
    op, dt, world, rank, m, n, k = c["op"], c["dt"], c["world"], c["rank"], c["m"], c["n"], c["k"]
    opts = dict(split=c["split"], deterministic=c["det"])
    if op in ("ar", "rs"):
        x = _values(c, synth.T_X, 0, (m, k), dt, -4, 4, 1.0)
        w, w64 = _weight(c)
        peers = [None if r == rank else _values(c, synth.T_PEER, r, (m, n), dt, -64, 64, _peer_sigma(c))
                 for r in range(world)]
        fn = tgc.matmul_all_reduce if op == "ar" else tgc.matmul_reduce_scatter
        y, p = fn(dev(x), dev(w), [dev(t) for t in peers], rank, trans_w=c["trans_w"], **opts)
        torch.cuda.synchronize()
        p_exact = oracle.matmul(f64(x, dt), w64)
        if op == "ar":
            rows = np.arange(m)
            assert tuple(y.shape) == (m, n)
        else:
            rows = rank * (m // world) + np.arange(m // world)
            assert tuple(y.shape) == (m // world, n)
        _check_reduce(c, y, p, p_exact, peers, rows, op)
    elif op in ("ag", "ag_v2"):
        shard = m // world
        shards = [_values(c, synth.T_X, r, (shard, k), dt, -4, 4, 1.0) for r in range(world)]
        w, w64 = _weight(c)
        peers = [None if r == rank else dev(shards[r]) for r in range(world)]
        out = tgc.allgather_matmul(dev(shards[rank]), peers, dev(w), rank, v2=(op == "ag_v2"),
                                   trans_w=c["trans_w"], **opts)
        torch.cuda.synchronize()
        y = out[0] if op == "ag_v2" else out
        g64 = oracle.allgather([f64(s, dt) for s in shards])
        y_ref = oracle.matmul(g64, w64)
        if op == "ag_v2":
            assert_bits_equal(out[1], np.vstack([raw(s) for s in shards]), "gathered")
        if c["integer"]:
            assert_bits_equal(y, encode_dtype(y_ref, dt), "y")
        else:
            assert_close(y, y_ref, dt, "y")
    else:
        mode, group = c["mode"], c["group"]
        wid = WID_SWEEP + c["i"]
        shape = {"per_tensor": (1,), "per_channel": (n,), "per_group": (k // max(group, 1), n)}[mode]
        if c["integer"]:
            x = synth.integers(wid, synth.T_X, 0, (m, k), -2, 2, "f16")
            q = synth.integers(wid, synth.T_W, 0, (k, n), -15, 15, "i8")
            s = synth.pow2_scales(wid, 0, shape)
        else:
            x = synth.normal(wid, synth.T_X, 0, (m, k), 1.0, "f16")
            q = synth.integers(wid, synth.T_W, 0, (k, n), -127, 127, "i8")
            s = synth.fp16_scales(wid, 0, shape)
        peers = [None if r == rank else _values(c, synth.T_PEER, r, (m, n), "f16", -64, 64,
                                                 0.6 * math.sqrt(k)) for r in range(world)]
        y, p = tgc.matmul_all_reduce_w8a16(dev(x), dev(q), dev(s), mode, [dev(t) for t in peers], rank,
                                           group_size=group, **opts)
        torch.cuda.synchronize()
        p_exact = oracle.matmul(f64(x, "f16"), oracle.dequant_weight(q.numpy(), f64(s, "f16"), mode, group))
        _check_reduce(c, y, p, p_exact, peers, np.arange(m), "w8a16")


# ------------------------------------------------------------------ MoE pair and weight gradient
def _draw_moe(i):
    r = random.Random(104729 * (i + 1))
    world = r.choice([1, 2, 4, 8])
    local = r.choice([1, 2, 4])
    pieces = r.choice([p for p in (1, 2, 4) if p * local <= 16 and p * local * world <= 128])
    return synth.MoeWorkload(f"sweep{i}", WID_SWEEP + 200 + i, r.choice(["bf16", "f16"]), world, world * local,
                             r.choice([1, 2]) if world * local > 1 else 1, r.randint(1, 600),
                             32 * r.randint(1, 16), 32 * r.randint(1, 16), pieces, rank=r.randrange(world))


MOE_CASES = [_draw_moe(i) for i in range(24)]


def _moe_id(wl):
    return (f"{wl.name}-{wl.dtype}-w{wl.world}r{wl.rank}-e{wl.experts}top{wl.topk}-p{wl.pieces}"
            f"-t{wl.tokens}-h{wl.hidden}-f{wl.ffn}")


@pytest.mark.parametrize("wl", MOE_CASES, ids=[_moe_id(w) for w in MOE_CASES])
def test_sweep_moe(wl):
    """Dispatch (all-to-all, then the grouped matmul) and combine (grouped
    matmul, then the all-to-all back) on seeded routings: received rows and
    returned rows bit for bit, matmul results normwise (Ampipe page, the
    expert all-to-all pair)."""
    from tests.test_gpu_moe import check_combine_copy, run_combine, run_dispatch
    counts = synth.moe_counts(wl)
    total = int(counts.sum())
    log(f"sweep moe {_moe_id(wl)}: {total} rows")
    sends = synth.moe_sends(wl, counts, wl.hidden)
    w1 = synth.moe_weights(wl, wl.hidden, wl.ffn)
    y, recv = run_dispatch(wl, counts, sends, w1)
    y_ref, recv_ref = oracle.alltoall_grouped_matmul([f64(s, wl.dtype) for s in sends], counts,
                                                     list(f64(w1, wl.dtype)))
    assert tuple(recv.shape) == (total, wl.hidden) and tuple(y.shape) == (total, wl.ffn)
    if total:
        assert_bits_equal(recv, encode_dtype(recv_ref, wl.dtype), "received rows")
        assert_close(y, y_ref, wl.dtype, "grouped matmul after the dispatch")
    h = synth.normal(wl.wid, synth.T_SEND, 100, (total, wl.ffn), 1.0, wl.dtype)
    w2 = synth.moe_weights(wl, wl.ffn, wl.hidden, which=1)
    outs, y_local = run_combine(wl, counts, h, w2)
    outs_ref, y2_ref = oracle.grouped_matmul_alltoall(f64(h, wl.dtype), counts, list(f64(w2, wl.dtype)))
    if total:
        assert_close(y_local, y2_ref, wl.dtype, "grouped matmul before the combine")
    for r in range(wl.world):
        assert outs[r].shape[0] == outs_ref[r].shape[0]
    check_combine_copy(y_local, outs, counts)


def _draw_wgrad(i):
    r = random.Random(15485863 * (i + 1))
    return dict(i=i, dt=r.choice(["bf16", "f16"]), m=32 * r.randint(1, 64), n=8 * r.randint(1, 130),
                k=8 * r.randint(1, 130), integer=r.random() < 0.5)


WGRAD_CASES = [_draw_wgrad(i) for i in range(24)]


@pytest.mark.parametrize("c", WGRAD_CASES,
                         ids=[f"{c['i']:02d}-{c['dt']}-{c['m']}x{c['n']}x{c['k']}-{'int' if c['integer'] else 'rnd'}"
                              for c in WGRAD_CASES])
def test_sweep_weight_grad(c):
    """dW = G^T dY (the backward of the sequence-parallel pair): exact bits for
    integer-valued inputs (|sum| <= 16 m < 2^24), normwise otherwise."""
    dt, m, n, k = c["dt"], c["m"], c["n"], c["k"]
    log(f"sweep weight_grad {dt} m={m} n={n} k={k}")
    wid = WID_SWEEP + 300 + c["i"]
    if c["integer"]:
        g = synth.integers(wid, synth.T_X, 0, (m, k), -4, 4, dt)
        dy = synth.integers(wid, synth.T_W, 0, (m, n), -4, 4, dt)
    else:
        g = synth.normal(wid, synth.T_X, 0, (m, k), 1.0, dt)
        dy = synth.normal(wid, synth.T_W, 0, (m, n), 1.0, dt)
    dw = tgc.weight_grad(dev(g), dev(dy))
    torch.cuda.synchronize()
    ref = oracle.weight_grad(f64(g, dt), f64(dy, dt))
    if c["integer"]:
        assert_bits_equal(dw, encode_dtype(ref, dt), "dW")
    else:
        assert_close(dw, ref, dt, "dW")
