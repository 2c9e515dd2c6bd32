"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/coc.h declares, plans chunks as documented, and rejects bad
arguments before anything is enqueued.

The error-path tests pass placeholder device addresses: validation must fail
before any HIP call.  They only run where no GPU is visible, so a validation
bug can never turn into a launch on fake pointers.
"""
import ctypes
import os
import re

import pytest

import tensor_gemm_collective_amd as tgc
from tensor_gemm_collective_amd import coc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coc.h")


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_have_gpu(), reason="placeholder pointers: host-only environment")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = tgc.lib()
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), f"{name} declared in coc.h but not exported"
    assert sorted(coc.EXPORTS) == names


def test_status_strings():
    L = tgc.lib()
    for code, name in coc.STATUS.items():
        assert L.coc_status_string(code).decode() == name


def test_mfma_loop_diagnostic_rejects_bad_arguments_on_the_host():
    """Validation happens before any HIP call (nothing is launched)."""
    L = tgc.lib()
    assert L.coc_diag_mfma_loop(None, 4096, None, 256, 1, 1, None) == 1          # COC_ERR_NULL
    assert L.coc_diag_mfma_loop(8, 4096, 40, 256, 1, 1, None) == 6              # COC_ERR_ALIGN
    assert L.coc_diag_mfma_loop(4096, 64, 8192, 256, 1, 1, None) == 3           # too few operand vectors
    assert L.coc_diag_mfma_loop(4096, 4096, 8192, 255, 1, 1, None) == 3         # out too small
    assert L.coc_diag_mfma_loop(4096, 4096, 8192, 256, 0, 1, None) == 3         # no workgroups
    assert L.coc_diag_mfma_loop(4096, 4096, 8192, 256, 1, 0, None) == 3         # no iterations
    assert "out must hold" in L.coc_last_error().decode() or "iters" in L.coc_last_error().decode()


def _rows_of(ch):
    rows = []
    for b in range(ch["nblk"]):
        start = ch["base"] + b * ch["stride"]
        rows.extend(range(start, start + ch["rows_per_blk"]))
    return rows


@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_plan_all_reduce_contiguous(split):
    m = 64
    chunks = tgc.plan(tgc.OP_MATMUL_ALL_REDUCE, m, 8, 3, split)
    assert len(chunks) == split
    seen = []
    for i, ch in enumerate(chunks):
        rows = _rows_of(ch)
        assert rows == list(range(i * m // split, (i + 1) * m // split))
        assert ch["red_base"] == rows[0] and ch["red_rows"] == len(rows) and ch["out_base"] == rows[0]
        seen += rows
    assert sorted(seen) == list(range(m))


@pytest.mark.parametrize("world,rank,split", [(8, 0, 4), (8, 5, 8), (2, 1, 2), (4, 2, 1), (1, 0, 4)])
def test_plan_reduce_scatter_interleaved(world, rank, split):
    m = 16 * world
    slice_rows = m // world
    chunks = tgc.plan(tgc.OP_MATMUL_REDUCE_SCATTER, m, world, rank, split)
    seen = []
    red = []
    for i, ch in enumerate(chunks):
        rows = _rows_of(ch)
        assert len(rows) == m // split
        # every chunk holds 1/split of every rank's slice
        for r in range(world):
            in_r = [x for x in rows if r * slice_rows <= x < (r + 1) * slice_rows]
            assert len(in_r) == slice_rows // split
        # the chunk's reduction rows are exactly its rows inside this rank's slice
        mine = [x for x in rows if rank * slice_rows <= x < (rank + 1) * slice_rows]
        assert mine == list(range(ch["red_base"], ch["red_base"] + ch["red_rows"]))
        assert ch["out_base"] == ch["red_base"] - rank * slice_rows
        seen += rows
        red += mine
    assert sorted(seen) == list(range(m))
    assert sorted(red) == list(range(rank * slice_rows, (rank + 1) * slice_rows))


@pytest.mark.parametrize("world,rank,split", [(8, 0, 4), (8, 5, 4), (8, 7, 8), (2, 1, 8), (4, 3, 2)])
def test_plan_allgather_starts_at_own_shard(world, rank, split):
    m = 16 * world
    shard = m // world
    chunks = tgc.plan(tgc.OP_ALLGATHER_MATMUL, m, world, rank, split)
    seen = []
    for ch in chunks:
        seen += _rows_of(ch)
    assert sorted(seen) == list(range(m))
    first = _rows_of(chunks[0])
    assert rank * shard in first          # own shard's first row is in the first chunk
    assert [c["order"] for c in chunks] == list(range(split))


@pytest.mark.parametrize("op,m,world,rank,split,status", [
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 8, 0, 3, "COC_ERR_SPLIT"),
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 8, 0, 16, "COC_ERR_SPLIT"),
    (tgc.OP_MATMUL_ALL_REDUCE, 66, 8, 0, 4, "COC_ERR_SHAPE"),
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 9, 0, 4, "COC_ERR_WORLD"),
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 0, 0, 4, "COC_ERR_WORLD"),
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 8, 8, 4, "COC_ERR_WORLD"),
    (tgc.OP_MATMUL_ALL_REDUCE, 64, 8, -1, 4, "COC_ERR_WORLD"),
    (tgc.OP_MATMUL_REDUCE_SCATTER, 60, 8, 0, 1, "COC_ERR_SHAPE"),
    (tgc.OP_MATMUL_REDUCE_SCATTER, 64, 8, 0, 16, "COC_ERR_SPLIT"),
    (tgc.OP_MATMUL_REDUCE_SCATTER, 32, 8, 0, 8, "COC_ERR_SHAPE"),   # slice 4 rows, split 8
    (tgc.OP_ALLGATHER_MATMUL, 24, 8, 0, 16, "COC_ERR_SPLIT"),
    (tgc.OP_ALLGATHER_MATMUL, 20, 8, 0, 4, "COC_ERR_SHAPE"),
    (tgc.OP_ALLGATHER_MATMUL, 48, 8, 0, 32, "COC_ERR_SPLIT"),
    (tgc.OP_ALLGATHER_MATMUL, 36, 8, 0, 4, "COC_ERR_SHAPE"),       # m % world
    (tgc.OP_ALLGATHER_MATMUL, 24, 8, 0, 16, "COC_ERR_SPLIT"),
])
def test_plan_rejects(op, m, world, rank, split, status):
    with pytest.raises(coc.CocError) as ei:
        tgc.plan(op, m, world, rank, split)
    assert ei.value.status_name == status
    assert tgc.lib().coc_last_error().decode() != ""


def test_workspace_bytes():
    L = tgc.lib()
    assert tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL, 4096, 7168, 8192, tgc.COC_BF16, 8, 4) == 4096 * 8192 * 2
    assert tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL_V2, 4096, 7168, 8192, tgc.COC_BF16, 8, 4) == 0
    assert tgc.workspace_bytes(tgc.OP_MATMUL_ALL_REDUCE, 4096, 7168, 8192, tgc.COC_BF16, 8, 4) == 0
    assert tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL, 4096, 7168, 8192, tgc.COC_F32, 8, 4) == 4096 * 8192 * 4
    assert tgc.workspace_bytes(tgc.OP_ALLGATHER_MATMUL, 4095, 7168, 8192, tgc.COC_BF16, 8, 4) == 0
    assert L.coc_last_error() is not None


# ------------------------------------------------------------------ op-level validation
A = 1 << 20   # placeholder device addresses, 16-byte aligned, far apart


def _addr(i):
    return A * (i + 1)


def _peers(world, rank, base=20):
    arr = (ctypes.c_void_p * world)()
    for r in range(world):
        arr[r] = None if r == rank else _addr(base + r) * 64
    return arr


def _ar(**kw):
    args = dict(x=_addr(1), w=_addr(2) * 16, y=_addr(3) * 256, p=_addr(4) * 1024, peers=_peers(8, 0),
                world=8, rank=0, m=64, n=64, k=64, dt=tgc.COC_BF16, split=4, det=0, tw=0)
    args.update(kw)
    L = tgc.lib()
    fn = L.coc_matmul_all_reduce_trans_w if args["tw"] else L.coc_matmul_all_reduce
    return fn(args["x"], args["w"], args["y"], args["p"], args["peers"],
              args["world"], args["rank"], args["m"], args["n"], args["k"],
              args["dt"], args["split"], args["det"], None, 0, None)


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(split=3), 2),
    (dict(split=0), 2),
    (dict(m=66), 3),
    (dict(n=60), 3),
    (dict(k=12), 3),
    (dict(m=1 << 31), 3),
    (dict(m=1 << 20, k=1 << 12), 3),
    (dict(world=9), 4),
    (dict(rank=8), 4),
    (dict(dt=7), 5),
    (dict(x=None), 1),
    (dict(w=None), 1),
    (dict(y=None), 1),
    (dict(p=None), 1),
    (dict(peers=None), 1),
    (dict(x=_addr(1) + 8), 6),
    (dict(y=_addr(3) * 256 + 2), 6),
    (dict(y=_addr(1)), 9),                   # y overlaps x
    (dict(p=_addr(3) * 256 + 4096), 9),      # partial_out overlaps y
    (dict(tw=1, dt=0), 5),                    # transposed weights: bf16 / fp16 only
    (dict(tw=1, k=48), 3),                    # transposed weights: k % 32 == 0
])
def test_all_reduce_rejects(kw, status):
    st = _ar(**kw)
    assert st == status, (st, tgc.lib().coc_last_error())
    assert tgc.lib().coc_last_error().decode() != ""


@no_gpu_only
def test_missing_peer_pointer_rejected():
    peers = _peers(8, 0)
    peers[3] = None
    assert _ar(peers=peers) == 1
    assert "peer_bufs[3]" in tgc.lib().coc_last_error().decode()


@no_gpu_only
def test_empty_problem_is_ok_and_touches_nothing():
    # m == 0: nothing to do, pointers may be NULL
    assert _ar(m=0, x=None, y=None, p=None, peers=None) == 0
    assert _ar(n=0, x=None, w=None, y=None, p=None, peers=None) == 0


@no_gpu_only
def test_w8a16_rejects():
    L = tgc.lib()

    def call(mode=tgc.COC_PER_GROUP, group=128, k=256, scales=_addr(9)):
        return L.coc_matmul_all_reduce_w8a16(_addr(1), _addr(2) * 16, scales, mode, group,
                                             _addr(3) * 256, _addr(4) * 1024, _peers(8, 0), 8, 0,
                                             64, 64, k, 4, 0, None, 0, None)
    assert call(mode=5) == 5
    assert call(group=0) == 3
    assert call(group=12) == 3
    assert call(group=96, k=256) == 3
    assert call(scales=None) == 1


@no_gpu_only
def test_allgather_rejects():
    L = tgc.lib()

    def call(gathered=None, ws=None, ws_bytes=0, m=64, split=4):
        return L.coc_allgather_matmul(_addr(1), _peers(8, 0), _addr(2) * 16, _addr(3) * 256, gathered,
                                      8, 0, m, 64, 64, tgc.COC_BF16, split, 0, ws, ws_bytes, None)
    assert call() == 7                                   # no workspace for the non-V2 form
    assert call(ws=_addr(5) * 512, ws_bytes=100) == 7    # too small
    assert call(ws=_addr(5) * 512 + 8, ws_bytes=1 << 20) == 6
    assert call(m=60) == 3
    assert call(split=5) == 2
    assert call(gathered=_addr(3) * 256) == 9            # gathered_out overlaps y


@no_gpu_only
def test_weight_grad_rejects():
    L = tgc.lib()

    def call(g=_addr(1), dy=_addr(2) * 16, dw=_addr(3) * 256, m=64, n=64, k=64, dt=tgc.COC_BF16):
        return L.coc_weight_grad(g, dy, dw, m, n, k, dt, None)
    assert call(m=48) == 3          # m % 32
    assert call(m=0) == 3
    assert call(n=60) == 3
    assert call(k=12) == 3
    assert call(dt=tgc.COC_F32) == 5
    assert call(g=None) == 1
    assert call(dw=_addr(1) + 16) == 9   # dw overlaps g
    assert call(dy=_addr(2) * 16 + 8) == 6


def _moe_counts(split, world, experts, value=3):
    import numpy as np
    c = np.full((split, world, experts), value, dtype=np.int64)
    return c


def test_expert_alltoall_rejects():
    """Argument checks of the MoE all-to-all entry points: each fails on the
    host, before anything is enqueued (no GPU needed)."""
    import numpy as np
    L = tgc.lib()

    def arr(c):
        c = np.asarray(c, dtype=np.int64)
        return (ctypes.c_int64 * max(c.size, 1))(*c.ravel().tolist())

    def dispatch(counts=None, world=2, rank=0, experts=2, split=2, n=32, k=64, dt=tgc.COC_BF16,
                 x_own=_addr(1), peers=None, w=_addr(3), y=_addr(4), recv=_addr(5), null_counts=False):
        c = _moe_counts(split, world, experts) if counts is None else counts
        peers = _peers(world, rank) if peers is None else peers
        return L.coc_alltoall_grouped_matmul(x_own, peers, None if null_counts else arr(c), w, y, recv,
                                             world, rank, experts, n, k, dt, split, None)

    def combine(counts=None, world=2, rank=0, experts=2, split=2, n=32, k=64, dt=tgc.COC_BF16,
                h=_addr(1), w=_addr(3), y_local=_addr(4), y_own=_addr(5), peers=None):
        c = _moe_counts(split, world, experts) if counts is None else counts
        peers = _peers(world, rank) if peers is None else peers
        return L.coc_grouped_matmul_alltoall(h, w, y_local, y_own, peers, arr(c), world, rank, experts,
                                             n, k, dt, split, None)

    assert dispatch(dt=tgc.COC_F32) == 5
    assert dispatch(k=48) == 3 and dispatch(n=12) == 3 and dispatch(k=0) == 3
    assert dispatch(split=0, counts=_moe_counts(1, 2, 2)) == 2
    assert dispatch(split=9, counts=_moe_counts(9, 2, 2)) == 2
    assert dispatch(world=9, counts=_moe_counts(2, 9, 2)) == 4
    assert dispatch(rank=2) == 4
    assert dispatch(experts=0, counts=_moe_counts(2, 2, 1)) == 3
    assert dispatch(experts=17, counts=_moe_counts(1, 2, 17), split=1) == 3
    bad = _moe_counts(2, 2, 2)
    bad[1, 1, 0] = -1
    assert dispatch(counts=bad) == 3
    assert dispatch(null_counts=True) == 1
    assert dispatch(x_own=None) == 1
    nopeer = _peers(2, 0)
    nopeer[1] = None
    assert dispatch(peers=nopeer) == 1
    # a source with no rows may pass NULL
    empty_src = _moe_counts(2, 2, 2)
    empty_src[:, 1, :] = 0
    assert dispatch(peers=nopeer, counts=empty_src, y=_addr(4) + 8) == 6   # fails later, on alignment
    assert dispatch(y=_addr(4) + 8) == 6
    assert dispatch(recv=_addr(4) + 16) == 9          # recv overlaps y
    assert dispatch(y=_addr(1) + 16) == 9             # y overlaps x_own
    # 8 pieces x 3 experts: 24 non-empty groups, more than a launch takes
    assert dispatch(split=8, experts=3, counts=_moe_counts(8, 2, 3)) == 3
    # nothing routed here: nothing to do, nothing touched
    assert dispatch(counts=_moe_counts(2, 2, 2, value=0), x_own=None, y=None, recv=None, w=None) == 0

    assert combine(dt=tgc.COC_F16, k=40) == 3
    assert combine(y_own=None) == 1
    assert combine(peers=nopeer) == 1
    assert combine(y_own=_addr(1) + 16) == 9          # y_own overlaps h
    assert combine(y_local=_addr(20 + 1) * 64) == 9   # y_local overlaps peer_out[1]
    assert combine(counts=_moe_counts(2, 2, 2, value=0), h=None, w=None, y_local=None, y_own=None) == 0
