"""Parity at the full workload sizes (one TP8 rank of BLOOM-7B, LLaMA2-70B,
BLOOM-176B, the w8A16 case), in the pipelined launch configurations the
benchmark uses.  Every element of every output is compared with the oracle
(float64 definitions, computed once per workload and shared by the cases):

* normwise relative error of y and partial_out over the whole tensor
  (5e-3 for bf16 / fp16);
* the gathered matrix bit for bit against the concatenated shards;
* in deterministic mode, y bit for bit against the oracle's fixed-order
  emulation of the stored partial_out and the peers' partials (ascending rank
  order, binary32 adds, one rounding), at every split, and identical over
  repeated runs;
* BLOOM-7B end to end with true shard peers: the other ranks' partials are
  the oracle's products of their own K shards, and y is compared with the
  unsplit full-K product X_full @ W_full (split-K invariance through the
  whole pipeline).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import assert_bits_equal, assert_close, encode_dtype, f64, log, raw

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _peers_full(wl, world, rank, dtype):
    return [None if r == rank else synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, dtype)
            for r in range(world)]


def _dev_list(ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _torch_from_oracle(x64, dtype):
    """A tensor holding the oracle's rounding of float64 values (an input the
    oracle computed, never the library)."""
    bits = encode_dtype(x64, dtype)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def assert_fixed_order(y, partial_out, peers, rank, dtype, what):
    """y bit for bit against the oracle's deterministic emulation, with this
    rank's own partial taken as the library stored it."""
    parts = [f64(partial_out, dtype) if r == rank else f64(p, dtype) for r, p in enumerate(peers)]
    want = oracle.reduce_fixed_order(parts, dtype)
    assert_bits_equal(y, encode_dtype(want, dtype), what)


# ------------------------------------------------------------------ BLOOM-7B all-reduce
@pytest.fixture(scope="module")
def bloom7b():
    wl = synth.WORKLOADS["bloom7b_ar"]
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    peers = _peers_full(wl, wl.world, 0, "bf16")
    y_ref, p_ref = oracle.matmul_all_reduce(f64(x, "bf16"), f64(w, "bf16"),
                                            [None if p is None else f64(p, "bf16") for p in peers], 0)
    return wl, x, w, peers, y_ref, p_ref


@pytest.mark.parametrize("split", [4, 2, 8])
def test_bloom7b_all_reduce(bloom7b, split):
    wl, x, w, peers, y_ref, p_ref = bloom7b
    log(f"BLOOM-7B AR bf16 {wl.m}x{wl.k}x{wl.n} split={split}")
    xd, wd, pd = x.to(DEV), w.to(DEV), _dev_list(peers)
    for det in (0, 1):
        y, p = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=det)
        torch.cuda.synchronize()
        assert_close(p, p_ref, "bf16", "partial_out")
        assert_close(y, y_ref, "bf16", f"y det={det}")
        if det:
            assert_fixed_order(y, p, peers, 0, "bf16", f"y det split={split} vs the fixed-order emulation")


def test_bloom7b_deterministic_across_splits(bloom7b):
    wl, x, w, peers, _, _ = bloom7b
    log("BLOOM-7B AR det bits across splits 2/4/8")
    xd, wd, pd = x.to(DEV), w.to(DEV), _dev_list(peers)
    ref = None
    for split in (2, 4, 8):
        y, _ = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=1)
        torch.cuda.synchronize()
        if ref is None:
            ref = y.clone()
        else:
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"split {split}"


@pytest.mark.parametrize("det", [0, 1])
def test_bloom7b_end_to_end_split_k(det):
    """The RowParallel layer of one TP8 group: rank r holds K shard r of
    X_full (2048 x 16384) and of W_full (16384 x 4096); the peers' partials
    are the oracle's bf16 products of their own shards.  y must match the
    unsplit product X_full @ W_full."""
    wl = synth.WORKLOADS["bloom7b_ar"]
    log(f"BLOOM-7B AR end to end with true shard peers det={det}")
    xs = [synth.normal(wl.wid, synth.T_X if r == 0 else synth.T_PEER, r, (wl.m, wl.k), wl.x_sigma, "bf16")
          for r in range(wl.world)]
    ws = [synth.normal(wl.wid, synth.T_W if r == 0 else synth.T_PEER_W, r, (wl.k, wl.n), wl.w_sigma, "bf16")
          for r in range(wl.world)]
    xf = [f64(t, "bf16") for t in xs]
    wf = [f64(t, "bf16") for t in ws]
    peers = [None] + [_torch_from_oracle(oracle.matmul(xf[r], wf[r]), "bf16") for r in range(1, wl.world)]
    y, p = tgc.matmul_all_reduce(xs[0].to(DEV), ws[0].to(DEV), _dev_list(peers), 0, split=4, deterministic=det)
    torch.cuda.synchronize()
    full = oracle.matmul(np.hstack(xf), np.vstack(wf))
    assert_close(y, full, "bf16", "y vs the unsplit full-K product")
    assert_close(p, oracle.matmul(xf[0], wf[0]), "bf16", "partial_out")


# ------------------------------------------------------------------ LLaMA2-70B all-gather matmul
@pytest.fixture(scope="module")
def llama_ag():
    wl = synth.WORKLOADS["llama70b_ag"]
    shard = wl.m // wl.world
    shards = [synth.normal(wl.wid, synth.T_PEER, r, (shard, wl.k), wl.x_sigma, "bf16") for r in range(wl.world)]
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    G = oracle.allgather([f64(s, "bf16") for s in shards])
    y_ref = oracle.matmul(G, f64(w, "bf16"))
    return wl, shards, w, G, y_ref


@pytest.fixture(scope="module")
def llama_ag_serial(llama_ag):
    """y of the serial form (split 1: every row gathered, then one matmul
    whose tiles each run all of k in one workgroup), as raw bits.  G is the
    same whatever the rank, so this is every rank's y."""
    wl, shards, w, _, _ = llama_ag
    sd = [s.to(DEV) for s in shards]
    y = tgc.allgather_matmul(sd[0], [None] + sd[1:], w.to(DEV), 0, split=1)
    torch.cuda.synchronize()
    return y.cpu().view(torch.int16)


@pytest.mark.parametrize("split", [2, 4, 8])
@pytest.mark.parametrize("rank", [0, 1, 3])
def test_llama_allgather_matmul(llama_ag, llama_ag_serial, split, rank):
    """V2's gathered matrix is the shards' bits; the plain op and V2 give the
    serial form's bits (the chunked one-launch pipeline, its fused copy and
    its tile order change when each tile runs, never what it adds).  The plain op's
    workspace starts as NaN: its tiles read the own shard's rows from the
    shard itself and it copies only the other rows, so no NaN may reach y.
    Ranks 0, 1, 3 at splits 2, 4, 8 put the own shard at the start, in the
    middle or at the end of its chunk, or make it the chunk."""
    wl, shards, w, _, y_ref = llama_ag
    log(f"LLaMA2-70B AG bf16 m={wl.m} k={wl.k} n={wl.n} split={split} rank={rank}")
    sd = [s.to(DEV) for s in shards]
    peers = [None if r == rank else sd[r] for r in range(wl.world)]
    wd = w.to(DEV)
    y, g = tgc.allgather_matmul(sd[rank], peers, wd, rank, split=split, v2=True)
    ws = torch.full((wl.m * wl.k * 2,), 0xFF, dtype=torch.uint8, device=DEV)   # bf16 NaN everywhere
    y1 = tgc.allgather_matmul(sd[rank], peers, wd, rank, split=split, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), torch.cat(sd).view(torch.int16)), "gathered rows differ"
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "V2 and plain results differ"
    assert torch.equal(y1.cpu().view(torch.int16), llama_ag_serial), "pipelined and serial results differ"
    assert_close(y, y_ref, "bf16", "y")


# ------------------------------------------------------------------ LLaMA2-70B backward of the pair
def test_llama_backward_pair(llama_ag):
    """The backward of the sequence-parallel MLP pair at full size: dW of the
    gate/up layer from V2's gathered G (8192 x 7168), and the dX of the down
    projection, AG(dY) @ W^T, with the 3584 x 8192 forward weight read
    transposed (reduction 8192, output 3584)."""
    wl, shards, w, G, _ = llama_ag
    rank = 2
    log(f"LLaMA2-70B backward: weight_grad {wl.k}x{wl.n} over m={wl.m}; AG dX with transposed weights")
    sd = [s.to(DEV) for s in shards]
    peers = [None if r == rank else sd[r] for r in range(wl.world)]
    _, g = tgc.allgather_matmul(sd[rank], peers, w.to(DEV), rank, split=4, v2=True)
    dy = synth.normal(wl.wid, synth.T_X, 9, (wl.m, wl.n), 1.0, "bf16")
    dw = tgc.weight_grad(g, dy.to(DEV))
    w_down = synth.normal(wl.wid, synth.T_W, 9, (3584, wl.k), 0.02, "bf16")       # forward RS weight, k x n
    dys = [synth.normal(wl.wid, synth.T_PEER, 9 + r, (wl.m // wl.world, wl.k), 1.0, "bf16") for r in range(wl.world)]
    dpeers = [None if r == rank else dys[r].to(DEV) for r in range(wl.world)]
    dx = tgc.allgather_matmul(dys[rank].to(DEV), dpeers, w_down.to(DEV), rank, split=4, trans_w=True)
    torch.cuda.synchronize()
    assert dw.shape == (wl.k, wl.n) and dx.shape == (wl.m, 3584)
    assert_close(dw, oracle.weight_grad(G, f64(dy, "bf16")), "bf16", "dW")
    DY = oracle.allgather([f64(d, "bf16") for d in dys])
    assert_close(dx, oracle.matmul(DY, f64(w_down, "bf16").T), "bf16", "dX")


# ------------------------------------------------------------------ LLaMA2-70B matmul reduce-scatter
@pytest.mark.parametrize("split", [4, 8])
def test_llama_allgather_matmul_nk_weights(llama_ag, llama_ag_serial, split):
    """The same all-gather product with W stored n x k (a Linear layer's out x
    in layout) through the transposed-weight entry point: its launch copies
    the gathered rows itself and takes the four-wave tile (448 tiles of
    256 x 256, k % 64 == 0), and must give the serial k x n form's bits."""
    wl, shards, w, _, y_ref = llama_ag
    rank = 2
    log(f"LLaMA2-70B AG bf16, W stored n x k, split={split} rank={rank}")
    sd = [s.to(DEV) for s in shards]
    wt = w.t().contiguous().to(DEV)
    y = tgc.allgather_matmul(sd[rank], [None if r == rank else sd[r] for r in range(wl.world)], wt, rank,
                             split=split, trans_w=True)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu().view(torch.int16), llama_ag_serial), "n x k weights: bits differ from k x n"
    assert_close(y, y_ref, "bf16", "y")


@pytest.fixture(scope="module")
def llama_rs():
    wl = synth.WORKLOADS["llama70b_rs"]
    rank = 5
    b = wl.m // wl.world
    x = synth.normal(wl.wid, synth.T_X, rank, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, rank, (wl.k, wl.n), wl.w_sigma, "bf16")
    slices = [None if r == rank else synth.normal(wl.wid, synth.T_PEER, r, (b, wl.n), wl.peer_sigma, "bf16")
              for r in range(wl.world)]
    p_ref = oracle.matmul(f64(x, "bf16"), f64(w, "bf16"))
    y_ref = p_ref[rank * b:(rank + 1) * b].copy()
    for s in slices:
        if s is not None:
            y_ref += f64(s, "bf16")
    return wl, rank, x, w, slices, p_ref, y_ref


def _rs_peers_dev(wl, rank, slices):
    b = wl.m // wl.world
    out = []
    for s in slices:
        if s is None:
            out.append(None)
            continue
        full = torch.full((wl.m, wl.n), float("nan"), dtype=torch.bfloat16, device=DEV)
        full[rank * b:(rank + 1) * b] = s.to(DEV)
        out.append(full)
    return out


def test_llama_reduce_scatter(llama_rs):
    wl, rank, x, w, slices, p_ref, y_ref = llama_rs
    b = wl.m // wl.world
    peers = _rs_peers_dev(wl, rank, slices)
    xd, wd = x.to(DEV), w.to(DEV)
    ref = None
    for split in (4, 8):
        log(f"LLaMA2-70B RS bf16 m={wl.m} k={wl.k} n={wl.n} split={split} rank={rank}")
        for det in (0, 1):
            y, p = tgc.matmul_reduce_scatter(xd, wd, peers, rank, split=split, deterministic=det)
            torch.cuda.synchronize()
            assert torch.isfinite(y.float()).all(), "NaN from an unread peer row leaked in"
            assert_close(y, y_ref, "bf16", f"y split={split} det={det}")
            assert_close(p, p_ref, "bf16", f"partial_out split={split} det={det}")
            if det:
                own = p[rank * b:(rank + 1) * b]
                assert_fixed_order(y, own, [None if s is None else s for s in slices], rank, "bf16",
                                   f"y det split={split} vs the fixed-order emulation")
                if ref is None:
                    ref = y.clone()
                else:
                    assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), "det bits differ across splits"


def test_llama_reduce_scatter_nk_weights(llama_rs):
    """The reduce-scatter product with W stored n x k through the transposed-
    weight entry point (its serial matmul runs alone on the four-wave tile):
    y and the partial must be the k x n call's bits."""
    wl, rank, x, w, slices, p_ref, y_ref = llama_rs
    peers = _rs_peers_dev(wl, rank, slices)
    xd = x.to(DEV)
    log(f"LLaMA2-70B RS bf16, W stored n x k, rank={rank}")
    y0, p0 = tgc.matmul_reduce_scatter(xd, w.to(DEV), peers, rank, split=4, deterministic=1)
    y1, p1 = tgc.matmul_reduce_scatter(xd, w.t().contiguous().to(DEV), peers, rank, split=4, deterministic=1,
                                       trans_w=True)
    torch.cuda.synchronize()
    assert torch.equal(p1.view(torch.int16), p0.view(torch.int16)), "partial: n x k and k x n bits differ"
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), "y: n x k and k x n bits differ"
    assert_close(y1, y_ref, "bf16", "y")


# ------------------------------------------------------------------ BLOOM-176B deterministic all-reduce
def test_bloom176b_deterministic():
    """The deterministic variant at full size: y bit for bit against the
    fixed-order emulation at splits 2, 4 and 8, identical over 10 runs, and
    y / partial_out against the exact float64 result over the whole tensor."""
    wl = synth.WORKLOADS["bloom176b_ar"]
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    peers = _peers_full(wl, wl.world, 0, "bf16")
    xd, wd, pd = x.to(DEV), w.to(DEV), _dev_list(peers)
    peers64 = [None if q is None else f64(q, "bf16") for q in peers]
    ref = None
    for split in (2, 4, 8):
        log(f"BLOOM-176B AR bf16 det m={wl.m} k={wl.k} n={wl.n} split={split}")
        runs = 10 if split == 4 else 1
        for run in range(runs):
            y, p = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=1)
            torch.cuda.synchronize()
            if ref is None:
                ref = (y.clone(), p.clone())
            else:
                assert torch.equal(y.view(torch.int16), ref[0].view(torch.int16)), f"y split={split} run={run}"
                assert torch.equal(p.view(torch.int16), ref[1].view(torch.int16)), f"partial split={split} run={run}"
        parts = [f64(p, "bf16")] + peers64[1:]
        assert_bits_equal(y, encode_dtype(oracle.reduce_fixed_order(parts, "bf16"), "bf16"),
                          f"y split={split} vs the fixed-order emulation")
    y_ref, p_ref = oracle.matmul_all_reduce(f64(x, "bf16"), f64(w, "bf16"), peers64, 0)
    assert_close(ref[1], p_ref, "bf16", "partial_out")
    assert_close(ref[0], y_ref, "bf16", "y")


# ------------------------------------------------------------------ w8A16
@pytest.mark.parametrize("mode", ["per_tensor", "per_channel", "per_group"])
def test_w8a16_full(mode):
    wl = synth.WORKLOADS["w8a16_ar"]
    log(f"w8A16 AR fp16 {mode} m={wl.m} k={wl.k} n={wl.n} split=4")
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), 1.0, "f16")
    q = synth.integers(wl.wid, synth.T_W, 0, (wl.k, wl.n), -127, 127, "i8")
    shape = {"per_tensor": (1,), "per_channel": (wl.n,), "per_group": (wl.k // wl.group, wl.n)}[mode]
    s = synth.fp16_scales(wl.wid, 0, shape)
    peers = _peers_full(wl, wl.world, 0, "f16")
    pd = _dev_list(peers)
    wt = oracle.dequant_weight(q.numpy(), f64(s, "f16"), mode, wl.group)
    y_ref, p_ref = oracle.matmul_all_reduce(f64(x, "f16"), wt, [None if t is None else f64(t, "f16") for t in peers], 0)
    for det in (0, 1):
        y, p = tgc.matmul_all_reduce_w8a16(x.to(DEV), q.to(DEV), s.to(DEV), mode, pd, 0,
                                           group_size=wl.group, split=4, deterministic=det)
        torch.cuda.synchronize()
        assert_close(p, p_ref, "f16", f"partial_out det={det}")
        assert_close(y, y_ref, "f16", f"y det={det}")
        if det:
            assert_fixed_order(y, p, peers, 0, "f16", "y det vs the fixed-order emulation")
