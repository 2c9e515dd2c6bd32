"""GPU parity of the MoE expert all-to-all + grouped matmul pair (Ampipe /
EP MC2) against the oracle: the received rows and the combine's copies bit
for bit, the grouped matmul within the bf16 / fp16 normwise tolerance, each
row's result independent of the sequence pieces and of earlier calls, the
edge cases (empty groups, a source with no rows, ragged tails), and the
Ampipe page's full-size scenario on sampled rows and columns."""
import numpy as np
import pytest
import torch

import oracle
import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import TOL, TORCH_DT, assert_bits_equal, assert_close, dev, encode_dtype, f64, log

pytestmark = pytest.mark.gpu


def src_offsets(counts):
    """(piece, source, expert) -> first row of that block in the source's rows."""
    P, W, E = counts.shape
    off = {}
    for r in range(W):
        row = 0
        for p in range(P):
            for e in range(E):
                off[(p, r, e)] = row
                row += int(counts[p, r, e])
    return off


def peers_of(sends, rank):
    return [None if (r == rank or s.shape[0] == 0) else dev(s) for r, s in enumerate(sends)]


def check_combine_copy(y_local, outs, counts):
    """Every returned row is, bit for bit, the grouped matmul's row of the same
    token (positions from the documented layouts)."""
    off = src_offsets(counts)
    idx = [[] for _ in outs]
    src = [[] for _ in outs]
    for j, (p, e, r, i) in enumerate(oracle.received_order(counts)):
        idx[r].append(off[(p, r, e)] + i)
        src[r].append(j)
    yl = y_local.cpu()
    for r, o in enumerate(outs):
        assert o.shape[0] == len(idx[r])
        if idx[r]:
            assert_bits_equal(o.cpu()[torch.tensor(idx[r])], yl[torch.tensor(src[r])], f"rows back to source {r}")


def run_dispatch(wl, counts, sends, w):
    y, recv = tgc.alltoall_grouped_matmul(dev(sends[wl.rank]), peers_of(sends, wl.rank), counts, dev(w), wl.rank)
    torch.cuda.synchronize()
    return y, recv


def run_combine(wl, counts, h, w):
    y_own, peer_out, y_local = tgc.grouped_matmul_alltoall(dev(h), dev(w), counts, wl.rank)
    torch.cuda.synchronize()
    return [y_own if r == wl.rank else peer_out[r] for r in range(wl.world)], y_local


@pytest.mark.parametrize("name", ["moe_small", "moe_ragged"])
def test_dispatch_matches_oracle(name):
    wl = synth.MOE_WORKLOADS[name]
    counts = synth.moe_counts(wl)
    sends = synth.moe_sends(wl, counts, wl.hidden)
    w = synth.moe_weights(wl, wl.hidden, wl.ffn)
    log(f"moe dispatch {name}: counts {counts.shape}, {int(counts.sum())} rows, k={wl.hidden} n={wl.ffn}")
    y, recv = run_dispatch(wl, counts, sends, w)
    y_ref, recv_ref = oracle.alltoall_grouped_matmul([f64(s, wl.dtype) for s in sends], counts,
                                                     list(f64(w, wl.dtype)))
    assert_bits_equal(recv, encode_dtype(recv_ref, wl.dtype), "received rows")
    assert_close(y, y_ref, wl.dtype, "grouped matmul after the dispatch")


@pytest.mark.parametrize("name", ["moe_small", "moe_ragged"])
def test_combine_matches_oracle(name):
    wl = synth.MOE_WORKLOADS[name]
    counts = synth.moe_counts(wl)
    total = int(counts.sum())
    k, n = wl.ffn, wl.hidden
    h = synth.normal(wl.wid, synth.T_SEND, 100, (total, k), 1.0, wl.dtype)
    w = synth.moe_weights(wl, k, n, which=1)
    log(f"moe combine {name}: {total} rows, k={k} n={n}")
    outs, y_local = run_combine(wl, counts, h, w)
    outs_ref, y_ref = oracle.grouped_matmul_alltoall(f64(h, wl.dtype), counts, list(f64(w, wl.dtype)))
    assert_close(y_local, y_ref, wl.dtype, "grouped matmul before the combine")
    for r in range(wl.world):
        if outs_ref[r].shape[0]:
            assert_close(outs[r], outs_ref[r], wl.dtype, f"rows back to source {r}")
    check_combine_copy(y_local, outs, counts)


def test_edge_groups():
    """Empty (piece, expert) groups, a source with no rows (NULL pointer), a
    one-row group, ragged row and column tails, the smallest k."""
    wl = synth.MoeWorkload("edge", 30, "bf16", 3, 9, 1, 0, 32, 200, 2, rank=2)
    counts = np.array([[[0, 1, 0], [0, 0, 0], [37, 0, 5]],
                       [[0, 0, 0], [0, 0, 0], [0, 290, 0]]], dtype=np.int64)
    sends = synth.moe_sends(wl, counts, 32)
    w1 = synth.moe_weights(wl, 32, 200)
    log("moe edge groups: dispatch")
    y, recv = run_dispatch(wl, counts, sends, w1)
    y_ref, recv_ref = oracle.alltoall_grouped_matmul([f64(s, "bf16") for s in sends], counts, list(f64(w1, "bf16")))
    assert_bits_equal(recv, encode_dtype(recv_ref, "bf16"), "received rows")
    assert_close(y, y_ref, "bf16", "grouped matmul")
    log("moe edge groups: combine")
    w2 = synth.moe_weights(wl, 32, 64, which=1)
    h = synth.normal(wl.wid, synth.T_SEND, 100, (int(counts.sum()), 32), 1.0, "bf16")
    outs, y_local = run_combine(wl, counts, h, w2)
    outs_ref, y2_ref = oracle.grouped_matmul_alltoall(f64(h, "bf16"), counts, list(f64(w2, "bf16")))
    assert_close(y_local, y2_ref, "bf16", "grouped matmul")
    assert outs[1].shape[0] == 0
    check_combine_copy(y_local, outs, counts)


def test_rows_independent_of_pieces():
    """The same tokens cut into 2 sequence pieces or left whole: each token's
    received row and both matmul results are bit-identical."""
    wl = synth.MOE_WORKLOADS["moe_small"]
    c2 = synth.moe_counts(wl)                    # 2 pieces
    s2 = synth.moe_sends(wl, c2, wl.hidden)
    w = synth.moe_weights(wl, wl.hidden, wl.ffn)
    P, W, E = c2.shape
    c1 = c2.sum(axis=0, keepdims=True)
    off2, off1 = src_offsets(c2), src_offsets(c1)
    # the same rows in the one-piece layout: expert-major, piece 0's before piece 1's
    tok1 = {}    # (r, e, index in one-piece block) -> (p, index in two-piece block)
    s1 = []
    for r in range(W):
        order = []
        for e in range(E):
            i1 = 0
            for p in range(P):
                for i in range(int(c2[p, r, e])):
                    order.append(off2[(p, r, e)] + i)
                    tok1[(r, e, i1)] = (p, i)
                    i1 += 1
        s1.append(s2[r][torch.tensor(order, dtype=torch.long)] if order else s2[r][:0])
    log("moe pieces: 2 pieces vs 1")
    y2, recv2 = run_dispatch(wl, c2, s2, w)
    y1, recv1 = run_dispatch(wl, c1, s1, w)
    j2 = {t: j for j, t in enumerate(oracle.received_order(c2))}
    perm = [j2[(tok1[(r, e, i)][0], e, r, tok1[(r, e, i)][1])] for (_, e, r, i) in oracle.received_order(c1)]
    perm = torch.tensor(perm, dtype=torch.long)
    assert_bits_equal(recv1, recv2.cpu()[perm], "received rows")
    assert_bits_equal(y1, y2.cpu()[perm], "grouped matmul")
    w2 = synth.moe_weights(wl, wl.ffn, wl.hidden, which=1)
    o2, _ = run_combine(wl, c2, y2, w2)
    o1, _ = run_combine(wl, c1, y1, w2)
    for r in range(W):
        back = []
        for e in range(E):
            for i in range(int(c1[0, r, e])):
                p, i2 = tok1[(r, e, i)]
                back.append(off2[(p, r, e)] + i2)
        assert_bits_equal(o1[r], o2[r].cpu()[torch.tensor(back, dtype=torch.long)], f"combined rows of source {r}")


def test_repeated_calls_through_the_same_buffers():
    """Two input sets alternate through the same output buffers: rows left
    from the previous call or counters out of step would show.  Every call
    matches the first call on its set bit for bit."""
    wl = synth.MOE_WORKLOADS["moe_ragged"]
    counts = synth.moe_counts(wl)
    total = int(counts.sum())
    sets = []
    for tag in (0, 1):
        s = [dev(x) for x in synth.moe_sends(synth.MoeWorkload(**{**wl.__dict__, "wid": 40 + tag}), counts,
                                              wl.hidden)]
        sets.append(s)
    w1 = dev(synth.moe_weights(wl, wl.hidden, wl.ffn))
    w2 = dev(synth.moe_weights(wl, wl.ffn, wl.hidden, which=1))
    y = torch.empty((total, wl.ffn), dtype=TORCH_DT[wl.dtype], device="cuda")
    recv = torch.empty((total, wl.hidden), dtype=TORCH_DT[wl.dtype], device="cuda")
    yl = torch.empty((total, wl.hidden), dtype=TORCH_DT[wl.dtype], device="cuda")
    rows = counts.sum(axis=(0, 2))
    outs = [torch.empty((int(rows[r]), wl.hidden), dtype=TORCH_DT[wl.dtype], device="cuda") for r in range(wl.world)]
    first = {}
    for it in range(6):
        s = sets[it % 2]
        log(f"moe repeated call {it}")
        tgc.alltoall_grouped_matmul(s[wl.rank], peers_of(s, wl.rank), counts, w1, wl.rank, y=y, recv_out=recv)
        tgc.grouped_matmul_alltoall(y, w2, counts, wl.rank, y_own=outs[wl.rank],
                                    peer_out=[None if r == wl.rank else outs[r] for r in range(wl.world)],
                                    y_local=yl)
        torch.cuda.synchronize()
        got = [recv.cpu(), y.cpu(), yl.cpu()] + [o.cpu() for o in outs]
        if it < 2:
            first[it] = got
        else:
            for a, b in zip(got, first[it % 2]):
                assert_bits_equal(a, b, f"call {it}")
    assert not torch.equal(first[0][1], first[1][1])


def test_ampipe_scenario_full_size():
    """The Ampipe page's scenario at full size (hidden 12288, ffn 49152, 8192
    tokens per rank, 4 experts, top 2, EP 2, 2 pieces): the received rows bit
    for bit against the oracle; both matmuls on sampled rows and columns in
    float64; the combine's copies bit for bit."""
    wl = synth.MOE_WORKLOADS["moe_ampipe"]
    counts = synth.moe_counts(wl)
    total = int(counts.sum())
    k, n = wl.hidden, wl.ffn
    g = torch.Generator(device="cuda").manual_seed(22)
    bf = torch.bfloat16
    rows = counts.sum(axis=(0, 2))
    sends = [torch.randn(int(rows[r]), k, device="cuda", generator=g).to(bf) for r in range(wl.world)]
    w1 = (torch.randn(wl.local, k, n, device="cuda", generator=g) * 0.02).to(bf)
    w2 = (torch.randn(wl.local, n, k, device="cuda", generator=g) * 0.02).to(bf)
    log(f"moe Ampipe scenario: {total} rows, dispatch k={k} n={n}, split {wl.pieces}")
    y1, recv = tgc.alltoall_grouped_matmul(sends[wl.rank], peers_of(sends, wl.rank), counts, w1, wl.rank)
    torch.cuda.synchronize()
    recv_ref = oracle.alltoall_dispatch([f64(s, "bf16") for s in sends], counts)
    assert_bits_equal(recv, encode_dtype(recv_ref, "bf16"), "received rows")
    order = oracle.received_order(counts)
    rng = np.random.default_rng(7)
    jr = np.sort(rng.choice(total, 48, replace=False))
    cols = np.sort(rng.choice(n, 96, replace=False))
    w1c = {e: f64(w1[e][:, torch.tensor(cols)], "bf16") for e in range(wl.local)}
    got = f64(y1[torch.tensor(jr, device="cuda")][:, torch.tensor(cols, device="cuda")], "bf16")
    ref = np.stack([recv_ref[j] @ w1c[order[j][1]] for j in jr])
    assert oracle.normwise_rel_error(got, ref) <= TOL["bf16"]
    del recv_ref
    log(f"moe Ampipe scenario: combine k={n} n={k}")
    h = torch.randn(total, n, device="cuda", generator=g).to(bf)
    outs, y_local = run_combine(wl, counts, h, w2)
    cols2 = np.sort(rng.choice(k, 96, replace=False))
    w2c = {e: f64(w2[e][:, torch.tensor(cols2)], "bf16") for e in range(wl.local)}
    hj = f64(h[torch.tensor(jr, device="cuda")], "bf16")
    got2 = f64(y_local[torch.tensor(jr, device="cuda")][:, torch.tensor(cols2, device="cuda")], "bf16")
    ref2 = np.stack([hj[i] @ w2c[order[j][1]] for i, j in enumerate(jr)])
    assert oracle.normwise_rel_error(got2, ref2) <= TOL["bf16"]
    check_combine_copy(y_local, outs, counts)
