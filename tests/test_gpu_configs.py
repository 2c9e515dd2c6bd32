"""Parity at the full workload sizes (one TP8 rank of BLOOM-7B, LLaMA2-70B,
BLOOM-176B, the w8A16 case), in the pipelined launch configurations the
benchmark uses.  The oracle computes sampled output rows one by one (float64);
whole-tensor properties are checked on the GPU: bit-exact gather, deterministic
bits identical across splits and repeated runs.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import TORCH_DT, assert_bits_equal, assert_close, f64, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


def sample_rows(m, chunks, n=48, seed=0):
    """Rows spread over every chunk, plus each chunk's first and last row."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, size=min(n, m), replace=False).tolist())
    step = m // chunks
    for c in range(chunks):
        rows.update((c * step, c * step + step - 1))
    return np.array(sorted(rows))


def _peers_full(wl, world, rank, dtype):
    return [None if r == rank else synth.normal(wl.wid, synth.T_PEER, r, (wl.m, wl.n), wl.peer_sigma, dtype)
            for r in range(world)]


def _f64_rows(t, rows, dtype):
    return f64(t[torch.as_tensor(rows)], dtype)


# ------------------------------------------------------------------ BLOOM-7B all-reduce
@pytest.fixture(scope="module")
def bloom7b():
    wl = synth.WORKLOADS["bloom7b_ar"]
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    peers = _peers_full(wl, wl.world, 0, "bf16")
    return wl, x, w, peers


@pytest.mark.parametrize("split", [4, 2, 8])
def test_bloom7b_all_reduce(bloom7b, split):
    wl, x, w, peers = bloom7b
    log(f"BLOOM-7B AR bf16 {wl.m}x{wl.k}x{wl.n} split={split}")
    xd, wd, pd = x.to(DEV), w.to(DEV), [None if p is None else p.to(DEV) for p in peers]
    rows = sample_rows(wl.m, split)
    wf = f64(w, "bf16")
    for det in (0, 1):
        y, p = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=det)
        torch.cuda.synchronize()
        y_ref, p_ref = oracle.matmul_all_reduce(
            _f64_rows(x, rows, "bf16"), wf, [None if q is None else _f64_rows(q, rows, "bf16") for q in peers], 0)
        assert_close(p[torch.as_tensor(rows)], p_ref, "bf16", "partial_out (sampled rows)")
        assert_close(y[torch.as_tensor(rows)], y_ref, "bf16", f"y det={det} (sampled rows)")


def test_bloom7b_deterministic_across_splits(bloom7b):
    wl, x, w, peers = bloom7b
    log("BLOOM-7B AR det bits across splits 2/4/8")
    xd, wd, pd = x.to(DEV), w.to(DEV), [None if p is None else p.to(DEV) for p in peers]
    ref = None
    for split in (2, 4, 8):
        y, _ = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=1)
        torch.cuda.synchronize()
        if ref is None:
            ref = y.clone()
        else:
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"split {split}"


# ------------------------------------------------------------------ LLaMA2-70B all-gather matmul
@pytest.fixture(scope="module")
def llama_ag():
    wl = synth.WORKLOADS["llama70b_ag"]
    shard = wl.m // wl.world
    shards = [synth.normal(wl.wid, synth.T_PEER, r, (shard, wl.k), wl.x_sigma, "bf16") for r in range(wl.world)]
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    return wl, shards, w


@pytest.mark.parametrize("split", [4, 8])
@pytest.mark.parametrize("rank", [0, 3])
def test_llama_allgather_matmul(llama_ag, split, rank):
    wl, shards, w = llama_ag
    log(f"LLaMA2-70B AG bf16 m={wl.m} k={wl.k} n={wl.n} split={split} rank={rank}")
    sd = [s.to(DEV) for s in shards]
    peers = [None if r == rank else sd[r] for r in range(wl.world)]
    wd = w.to(DEV)
    y, g = tgc.allgather_matmul(sd[rank], peers, wd, rank, split=split, v2=True)
    y1 = tgc.allgather_matmul(sd[rank], peers, wd, rank, split=split)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), torch.cat(sd).view(torch.int16)), "gathered rows differ"
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "V2 and plain results differ"
    rows = sample_rows(wl.m, split, seed=split + rank)
    g_rows = oracle.allgather([f64(s, "bf16") for s in shards])[rows]
    assert_close(y[torch.as_tensor(rows)], oracle.matmul(g_rows, f64(w, "bf16")), "bf16", "y (sampled rows)")


# ------------------------------------------------------------------ LLaMA2-70B backward of the pair
def test_llama_backward_pair(llama_ag):
    """The backward of the sequence-parallel MLP pair at full size: dW of the
    gate/up layer from V2's gathered G (8192 x 7168), and the dX of the down
    projection, AG(dY) @ W^T, with the 3584 x 8192 forward weight read
    transposed (reduction 8192, output 3584)."""
    wl, shards, w = llama_ag
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
    rows = sample_rows(wl.k, 8, n=24, seed=21)
    G = oracle.allgather([f64(s, "bf16") for s in shards])
    assert_close(dw[torch.as_tensor(rows)], oracle.weight_grad(G[:, rows], f64(dy, "bf16")), "bf16", "dW rows")
    rows = sample_rows(wl.m, 4, n=24, seed=22)
    DY = oracle.allgather([f64(d, "bf16") for d in dys])
    assert_close(dx[torch.as_tensor(rows)], oracle.matmul(DY[rows], f64(w_down, "bf16").T), "bf16", "dX rows")


# ------------------------------------------------------------------ LLaMA2-70B matmul reduce-scatter
@pytest.fixture(scope="module")
def llama_rs():
    wl = synth.WORKLOADS["llama70b_rs"]
    rank = 5
    b = wl.m // wl.world
    x = synth.normal(wl.wid, synth.T_X, rank, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, rank, (wl.k, wl.n), wl.w_sigma, "bf16")
    slices = [None if r == rank else synth.normal(wl.wid, synth.T_PEER, r, (b, wl.n), wl.peer_sigma, "bf16")
              for r in range(wl.world)]
    return wl, rank, x, w, slices


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
    wl, rank, x, w, slices = llama_rs
    b = wl.m // wl.world
    peers = _rs_peers_dev(wl, rank, slices)
    xd, wd = x.to(DEV), w.to(DEV)
    wf = f64(w, "bf16")
    local = sample_rows(b, 8, n=40, seed=7)
    ref = None
    for split in (4, 8):
        log(f"LLaMA2-70B RS bf16 m={wl.m} k={wl.k} n={wl.n} split={split} rank={rank}")
        for det in (0, 1):
            y, p = tgc.matmul_reduce_scatter(xd, wd, peers, rank, split=split, deterministic=det)
            torch.cuda.synchronize()
            assert torch.isfinite(y.float()).all(), "NaN from an unread peer row leaked in"
            # rows j of this rank's slice are rows rank*b + j of the all-reduced sum
            glob = rank * b + local
            y_ref, _ = oracle.matmul_all_reduce(
                _f64_rows(x, glob, "bf16"), wf,
                [None if sl is None else _f64_rows(sl, local, "bf16") for sl in slices], rank)
            assert_close(y[torch.as_tensor(local)], y_ref, "bf16", f"y split={split} det={det}")
            prow = sample_rows(wl.m, split, n=24, seed=split)
            assert_close(p[torch.as_tensor(prow)], oracle.matmul(_f64_rows(x, prow, "bf16"), wf), "bf16",
                         "partial_out")
            if det:
                if ref is None:
                    ref = y.clone()
                else:
                    assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), "det bits differ across splits"


# ------------------------------------------------------------------ BLOOM-176B deterministic all-reduce
def test_bloom176b_deterministic():
    wl = synth.WORKLOADS["bloom176b_ar"]
    log(f"BLOOM-176B AR bf16 det m={wl.m} k={wl.k} n={wl.n}")
    x = synth.normal(wl.wid, synth.T_X, 0, (wl.m, wl.k), wl.x_sigma, "bf16")
    w = synth.normal(wl.wid, synth.T_W, 0, (wl.k, wl.n), wl.w_sigma, "bf16")
    peers = _peers_full(wl, wl.world, 0, "bf16")
    xd, wd, pd = x.to(DEV), w.to(DEV), [None if p is None else p.to(DEV) for p in peers]
    ref = None
    for split in (2, 4, 8):
        runs = 10 if split == 4 else 1
        for run in range(runs):
            y, p = tgc.matmul_all_reduce(xd, wd, pd, 0, split=split, deterministic=1)
            torch.cuda.synchronize()
            if ref is None:
                ref = (y.clone(), p.clone())
            else:
                assert torch.equal(y.view(torch.int16), ref[0].view(torch.int16)), f"y split={split} run={run}"
                assert torch.equal(p.view(torch.int16), ref[1].view(torch.int16)), f"partial split={split} run={run}"
    rows = sample_rows(wl.m, 8, n=32, seed=3)
    y_ref, p_ref = oracle.matmul_all_reduce(
        _f64_rows(x, rows, "bf16"), f64(w, "bf16"), [None if q is None else _f64_rows(q, rows, "bf16") for q in peers], 0)
    assert_close(ref[1][torch.as_tensor(rows)], p_ref, "bf16", "partial_out (sampled rows)")
    assert_close(ref[0][torch.as_tensor(rows)], y_ref, "bf16", "y (sampled rows)")


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
    y, p = tgc.matmul_all_reduce_w8a16(x.to(DEV), q.to(DEV), s.to(DEV), mode,
                                       [None if t is None else t.to(DEV) for t in peers], 0,
                                       group_size=wl.group, split=4)
    torch.cuda.synchronize()
    rows = sample_rows(wl.m, 4, n=40, seed=11)
    wt = oracle.dequant_weight(q.numpy(), f64(s, "f16"), mode, wl.group)
    y_ref, p_ref = oracle.matmul_all_reduce(
        _f64_rows(x, rows, "f16"), wt, [None if t is None else _f64_rows(t, rows, "f16") for t in peers], 0)
    assert_close(p[torch.as_tensor(rows)], p_ref, "f16", "partial_out (sampled rows)")
    assert_close(y[torch.as_tensor(rows)], y_ref, "f16", "y (sampled rows)")
