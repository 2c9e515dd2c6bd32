"""Graph capture of the fused ops: each op is captured into a HIP graph
(torch.cuda.CUDAGraph) and replayed several times, with the inputs changed
between replays and eager calls of the same op on the same stream in between.
Every replay must give the bits of the eager call on the same inputs (a
replay that reused the hand-over state of the capture would read unfinished
chunks).  The MoE all-to-all pair and a first call on an uncaptured stream are
refused with COC_ERR_CAPTURE, before anything is enqueued."""
import pytest
import torch

import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import synth
from tests._util import TORCH_DT, assert_bits_equal, dev, log, raw

pytestmark = pytest.mark.gpu

WID = 140


def _warm_and_capture(fn, stream):
    """One eager call on `stream` (sets up the library's context for it), then the
    same call captured into a graph on it."""
    with torch.cuda.stream(stream):
        fn()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, stream, x, sources, outs, eager):
    """For each source: copy it into x, replay, compare outs with an eager call
    on the same stream (fresh outputs) bit for bit."""
    for it, src in enumerate(sources):
        x.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            want = eager()   # fresh outputs: outs still hold the replay's results
        torch.cuda.synchronize()
        for i, (o, b) in enumerate(zip(outs, want)):
            assert_bits_equal(o, b, f"replay {it}, output {i}")


@pytest.mark.parametrize("det", [0, 1])
@pytest.mark.parametrize("op", ["ar", "rs"])
def test_compute_first_graph_replay(op, det):
    log(f"graph replay {op} det={det}")
    dtype, m, n, k, world, rank, split = "bf16", 1024, 512, 256, 8, 5, 4
    b = m // world
    xs = [dev(synth.normal(WID, synth.T_X, i, (m, k), 1.0, dtype)) for i in range(2)]
    w = dev(synth.normal(WID, synth.T_W, rank, (k, n), 0.05, dtype))
    peers = [None if q is None else dev(q) for q in synth.peers_random(WID, world, rank, (m, n), 0.4, dtype)]
    x = xs[0].clone()
    rows = m if op == "ar" else b
    y = torch.empty((rows, n), dtype=TORCH_DT[dtype], device="cuda")
    p = torch.empty((m, n), dtype=TORCH_DT[dtype], device="cuda")
    fn = tgc.matmul_all_reduce if op == "ar" else tgc.matmul_reduce_scatter

    def call(xin, yo, po):
        return fn(xin, w, peers, rank, y=yo, partial_out=po, split=split, deterministic=det)

    s = torch.cuda.Stream()
    g = _warm_and_capture(lambda: call(x, y, p), s)
    _replay_and_check(g, s, x, [xs[1], xs[0], xs[1]], [y, p],
                      lambda: [raw(t) for t in call(x.clone(), None, None)])


@pytest.mark.parametrize("v2", [False, True])
def test_allgather_graph_replay(v2):
    log(f"graph replay AG v2={v2}")
    dtype, m, n, k, world, rank, split = "bf16", 1024, 640, 256, 8, 2, 4
    shard = m // world
    shards = [dev(synth.normal(WID + 1, synth.T_PEER, r, (shard, k), 1.0, dtype)) for r in range(world)]
    other = dev(synth.normal(WID + 1, synth.T_X, 0, (shard, k), 1.0, dtype))
    w = dev(synth.normal(WID + 1, synth.T_W, 0, (k, n), 0.05, dtype))
    peers = [None if r == rank else shards[r] for r in range(world)]
    x = shards[rank].clone()
    y = torch.empty((m, n), dtype=TORCH_DT[dtype], device="cuda")
    gat = torch.empty((m, k), dtype=TORCH_DT[dtype], device="cuda") if v2 else None
    ws = None if v2 else torch.empty(tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL, m, n, k, tgc.COC_BF16, world,
                                                         split), dtype=torch.uint8, device="cuda")

    def call(xin, yo, go, wso):
        r = tgc.allgather_matmul(xin, peers, w, rank, y=yo, gathered_out=go, v2=v2, ws=wso, split=split)
        return list(r) if v2 else [r]

    s = torch.cuda.Stream()
    g = _warm_and_capture(lambda: call(x, y, gat, ws), s)
    _replay_and_check(g, s, x, [other, shards[rank], other], [y, gat] if v2 else [y],
                      lambda: [raw(t) for t in call(x.clone(), None, None, None)])


def test_w8a16_graph_replay():
    log("graph replay w8a16")
    m, n, k, world, rank, split, grp = 1024, 512, 256, 8, 1, 4, 128
    xs = [dev(synth.normal(WID + 2, synth.T_X, i, (m, k), 1.0, "f16")) for i in range(2)]
    q = dev(synth.integers(WID + 2, synth.T_W, rank, (k, n), -127, 127, "i8"))
    sc = dev(synth.fp16_scales(WID + 2, rank, (k // grp, n)))
    peers = [None if t is None else dev(t) for t in synth.peers_random(WID + 2, world, rank, (m, n), 20.0, "f16")]
    x = xs[0].clone()
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    p = torch.empty((m, n), dtype=torch.float16, device="cuda")

    def call(xin, yo, po):
        return tgc.matmul_all_reduce_w8a16(xin, q, sc, "per_group", peers, rank, group_size=grp, y=yo,
                                           partial_out=po, split=split, deterministic=1)

    s = torch.cuda.Stream()
    g = _warm_and_capture(lambda: call(x, y, p), s)
    _replay_and_check(g, s, x, [xs[1], xs[0]], [y, p], lambda: [raw(t) for t in call(x.clone(), None, None)])


def test_capture_refusals():
    log("graph capture refusals")
    # a first call on a stream sets up its context and cannot be captured
    m, n, k, world, rank = 256, 256, 64, 2, 0
    x = dev(synth.normal(WID + 3, synth.T_X, 0, (m, k), 1.0, "bf16"))
    w = dev(synth.normal(WID + 3, synth.T_W, 0, (k, n), 0.05, "bf16"))
    peers = [None, dev(synth.normal(WID + 3, synth.T_PEER, 1, (m, n), 0.4, "bf16"))]
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    p = torch.empty_like(y)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(tgc.CocError) as ei:
        with torch.cuda.graph(g, stream=s):
            tgc.matmul_all_reduce(x, w, peers, rank, y=y, partial_out=p, split=4)
    assert ei.value.status_name == "COC_ERR_CAPTURE"
    torch.cuda.synchronize()

    # the MoE pair works through device counters only
    wl = synth.MOE_WORKLOADS["moe_small"]
    counts = synth.moe_counts(wl)
    sends = synth.moe_sends(wl, counts, wl.hidden)
    wm = dev(synth.moe_weights(wl, wl.hidden, wl.ffn))
    own = dev(sends[wl.rank])
    mp = [None if (r == wl.rank or t.shape[0] == 0) else dev(t) for r, t in enumerate(sends)]
    s2 = torch.cuda.Stream()
    with torch.cuda.stream(s2):
        ym, recv = tgc.alltoall_grouped_matmul(own, mp, counts, wm, wl.rank)   # eager: sets up s2
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(tgc.CocError) as ei:
        with torch.cuda.graph(g2, stream=s2):
            tgc.alltoall_grouped_matmul(own, mp, counts, wm, wl.rank, y=ym, recv_out=recv)
    assert ei.value.status_name == "COC_ERR_CAPTURE"
    torch.cuda.synchronize()


def test_second_call_in_one_capture_refused():
    """One capture holds at most one call of the library: a second call while
    the same capture is open (here the reduce-scatter after the all-reduce) is
    refused with COC_ERR_CAPTURE and enqueues nothing.  The graph then holds
    the first call alone and replays it exactly; the refused call's outputs
    are never written."""
    log("second call in one capture refused")
    dtype, m, n, k, world, rank, split = "bf16", 1024, 512, 256, 8, 3, 4
    x = dev(synth.normal(WID + 4, synth.T_X, 0, (m, k), 1.0, dtype))
    w = dev(synth.normal(WID + 4, synth.T_W, rank, (k, n), 0.05, dtype))
    peers = [None if q is None else dev(q) for q in synth.peers_random(WID + 4, world, rank, (m, n), 0.4, dtype)]
    y = torch.empty((m, n), dtype=TORCH_DT[dtype], device="cuda")
    p = torch.empty((m, n), dtype=TORCH_DT[dtype], device="cuda")
    y2 = torch.zeros((m // world, n), dtype=TORCH_DT[dtype], device="cuda")
    p2 = torch.zeros((m, n), dtype=TORCH_DT[dtype], device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        want_y, want_p = tgc.matmul_all_reduce(x, w, peers, rank, split=split, deterministic=1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tgc.matmul_all_reduce(x, w, peers, rank, y=y, partial_out=p, split=split, deterministic=1)
        with pytest.raises(tgc.CocError) as ei:
            tgc.matmul_reduce_scatter(x, w, peers, rank, y=y2, partial_out=p2, split=split, deterministic=1)
    assert ei.value.status_name == "COC_ERR_CAPTURE"
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(y, want_y, "captured all-reduce y")
        assert_bits_equal(p, want_p, "captured all-reduce partial")
    assert not y2.any() and not p2.any(), "the refused call wrote its outputs"
