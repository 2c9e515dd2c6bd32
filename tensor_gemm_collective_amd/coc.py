"""ctypes binding of libcoc.so (include/coc.h).

Argument marshalling only: every step of an op runs in the library's HIP
kernels.  torch provides device memory and the current stream.  The
library must have been built (``__graft_entry__.build()``); loading fails
loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoc.so")

# enums of include/coc.h
COC_F32, COC_F16, COC_BF16 = 0, 1, 2
COC_PER_TENSOR, COC_PER_CHANNEL, COC_PER_GROUP = 0, 1, 2
OP_MATMUL_ALL_REDUCE = 0
OP_MATMUL_REDUCE_SCATTER = 1
OP_ALLGATHER_MATMUL = 2
OP_ALLGATHER_MATMUL_V2 = 3
OP_MATMUL_ALL_REDUCE_W8A16 = 4
STATUS = {
    0: "COC_OK", 1: "COC_ERR_NULL", 2: "COC_ERR_SPLIT", 3: "COC_ERR_SHAPE", 4: "COC_ERR_WORLD",
    5: "COC_ERR_DTYPE", 6: "COC_ERR_ALIGN", 7: "COC_ERR_WORKSPACE", 8: "COC_ERR_HIP",
    9: "COC_ERR_ALIAS", 10: "COC_ERR_CAPTURE", 11: "COC_ERR_TIMEOUT",
}
QUANT_MODES = {"per_tensor": COC_PER_TENSOR, "per_channel": COC_PER_CHANNEL, "per_group": COC_PER_GROUP}
KCLASS = ("gemm", "reduce", "gather")

# exported symbols, as declared in include/coc.h
EXPORTS = (
    "coc_matmul_all_reduce", "coc_matmul_reduce_scatter", "coc_allgather_matmul",
    "coc_matmul_all_reduce_w8a16", "coc_matmul_all_reduce_trans_w", "coc_matmul_reduce_scatter_trans_w",
    "coc_allgather_matmul_trans_w", "coc_allgather_matmul_noalloc", "coc_weight_grad", "coc_alltoall_grouped_matmul",
    "coc_grouped_matmul_alltoall", "coc_workspace_bytes", "coc_status_string",
    "coc_last_error", "coc_check_waits", "coc_plan", "coc_profile_enable", "coc_profile_read",
    "coc_profile_records", "coc_profile_stamps", "coc_profile_stamp_count", "coc_diag_mfma_loop",
)


class CocError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


class Chunk(ctypes.Structure):
    _fields_ = [
        ("base", ctypes.c_int64), ("stride", ctypes.c_int64), ("rows_per_blk", ctypes.c_int64),
        ("nblk", ctypes.c_int32), ("order", ctypes.c_int32), ("red_base", ctypes.c_int64),
        ("out_base", ctypes.c_int64), ("red_rows", ctypes.c_int64),
    ]


_lib = None
_vp = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libcoc.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads torch's libamdhip64 first; ours resolves to it

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    # world, rank, m, n, k, dt, split, deterministic, ws, ws_bytes, stream
    common = [_i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _sz, _vp]
    for f in ("coc_matmul_all_reduce", "coc_matmul_reduce_scatter", "coc_matmul_all_reduce_trans_w",
              "coc_matmul_reduce_scatter_trans_w"):
        getattr(L, f).argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(_vp)] + common
    for f in ("coc_allgather_matmul", "coc_allgather_matmul_trans_w"):
        getattr(L, f).argtypes = [_vp, ctypes.POINTER(_vp), _vp, _vp, _vp] + common
    L.coc_matmul_all_reduce_w8a16.argtypes = [
        _vp, _vp, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(_vp), _i32, _i32, _i64, _i64, _i64,
        _i32, _i32, _vp, _sz, _vp]
    L.coc_weight_grad.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]
    moe_tail = [ctypes.POINTER(_i64), _i32, _i32, _i32, _i64, _i64, _i32, _i32, _vp]
    L.coc_alltoall_grouped_matmul.argtypes = [_vp, ctypes.POINTER(_vp)] + moe_tail[:1] + [_vp, _vp, _vp] + moe_tail[1:]
    L.coc_grouped_matmul_alltoall.argtypes = [_vp, _vp, _vp, _vp, ctypes.POINTER(_vp)] + moe_tail
    for f in ("coc_matmul_all_reduce", "coc_matmul_reduce_scatter", "coc_allgather_matmul",
              "coc_matmul_all_reduce_trans_w", "coc_matmul_reduce_scatter_trans_w",
              "coc_allgather_matmul_trans_w", "coc_matmul_all_reduce_w8a16", "coc_weight_grad",
              "coc_alltoall_grouped_matmul", "coc_grouped_matmul_alltoall"):
        getattr(L, f).restype = _i32
    L.coc_allgather_matmul_noalloc.argtypes = [_vp, ctypes.POINTER(_vp), _vp, _vp, _i32, _i32, _i64, _i64, _i64,
                                               _i32, _i32, _i32, _vp]
    L.coc_allgather_matmul_noalloc.restype = _i32
    L.coc_check_waits.argtypes = [_vp]
    L.coc_check_waits.restype = _i32
    L.coc_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64, _i32, _i32, _i32]
    L.coc_workspace_bytes.restype = _sz
    L.coc_status_string.argtypes = [_i32]
    L.coc_status_string.restype = ctypes.c_char_p
    L.coc_last_error.argtypes = []
    L.coc_last_error.restype = ctypes.c_char_p
    L.coc_plan.argtypes = [_i32, _i64, _i32, _i32, _i32, ctypes.POINTER(Chunk), _i32, ctypes.POINTER(_i32)]
    L.coc_plan.restype = _i32
    L.coc_profile_enable.argtypes = [_i32]
    L.coc_profile_enable.restype = None
    L.coc_profile_stamps.argtypes = [_vp, _i64]
    L.coc_profile_stamps.restype = None
    L.coc_profile_stamp_count.argtypes = []
    L.coc_profile_stamp_count.restype = _i64
    L.coc_diag_mfma_loop.argtypes = [_vp, _sz, _vp, _sz, _i32, _i32, _vp]
    L.coc_diag_mfma_loop.restype = _i32
    L.coc_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64),
                                   ctypes.POINTER(ctypes.c_double)]
    L.coc_profile_read.restype = _i32
    dp = ctypes.POINTER(ctypes.c_double)
    L.coc_profile_records.argtypes = [ctypes.POINTER(_i32), dp, dp, dp, _i32, ctypes.POINTER(_i32)]
    L.coc_profile_records.restype = _i32
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise CocError(status, lib().coc_last_error().decode())


# ------------------------------------------------------------------ marshalling
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: COC_F32, torch.float16: COC_F16, torch.bfloat16: COC_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (row-major)")
    return t.data_ptr()


def _peer_array(peers: Sequence, rank: int):
    arr = (_vp * len(peers))()
    for r, p in enumerate(peers):
        arr[r] = None if (r == rank or p is None) else _ptr(p)
    return arr


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _empty(shape, like):
    import torch
    return torch.empty(shape, dtype=like.dtype, device=like.device)


# ------------------------------------------------------------------ ops
def _wdims(w, trans_w):
    """(k, n) of a weight given k x n, or n x k when trans_w."""
    return (w.shape[1], w.shape[0]) if trans_w else (w.shape[0], w.shape[1])


def matmul_all_reduce(x, w, peers, rank, *, y=None, partial_out=None, split=4, deterministic=False,
                      trans_w=False, stream=None):
    """MATMUL_ALL_REDUCE: returns (y, partial_out).  peers[r] (r != rank) are m x n partials.
    trans_w: w is n x k (the product uses its transpose)."""
    m, k = x.shape
    n = _wdims(w, trans_w)[1]
    y = _empty((m, n), x) if y is None else y
    partial_out = _empty((m, n), x) if partial_out is None else partial_out
    fn = lib().coc_matmul_all_reduce_trans_w if trans_w else lib().coc_matmul_all_reduce
    _check(fn(
        _ptr(x), _ptr(w), _ptr(y), _ptr(partial_out), _peer_array(peers, rank), len(peers), rank,
        m, n, k, _dtype_code(x), split, int(bool(deterministic)), None, 0, _stream(stream, x.device)))
    return y, partial_out


def matmul_reduce_scatter(x, w, peers, rank, *, y=None, partial_out=None, split=4,
                          deterministic=False, trans_w=False, stream=None):
    """MATMUL_REDUCE_SCATTER: returns (y, partial_out); y is (m/world) x n.
    trans_w: w is n x k (the product uses its transpose)."""
    m, k = x.shape
    n = _wdims(w, trans_w)[1]
    world = len(peers)
    y = _empty((m // world, n), x) if y is None else y
    partial_out = _empty((m, n), x) if partial_out is None else partial_out
    fn = lib().coc_matmul_reduce_scatter_trans_w if trans_w else lib().coc_matmul_reduce_scatter
    _check(fn(
        _ptr(x), _ptr(w), _ptr(y), _ptr(partial_out), _peer_array(peers, rank), world, rank,
        m, n, k, _dtype_code(x), split, int(bool(deterministic)), None, 0, _stream(stream, x.device)))
    return y, partial_out


def allgather_matmul(x_shard, peers, w, rank, *, y=None, gathered_out=None, v2=False, ws=None,
                     split=4, deterministic=False, trans_w=False, stream=None):
    """ALL_GATHER_MATMUL (v2=False) or _V2 (v2=True, also returns the gathered matrix).

    Returns y, or (y, gathered) for V2.  peers[r] (r != rank) are (m/world) x k shards.
    trans_w: w is n x k (the product uses its transpose)."""
    import torch
    world = len(peers)
    shard, k = x_shard.shape
    m = shard * world
    n = _wdims(w, trans_w)[1]
    y = _empty((m, n), x_shard) if y is None else y
    if v2 and gathered_out is None:
        gathered_out = _empty((m, k), x_shard)
    ws_bytes = 0
    if not v2:
        need = workspace_bytes(OP_ALLGATHER_MATMUL, m, n, k, _dtype_code(x_shard), world, split)
        if ws is None and need:
            ws = torch.empty(need, dtype=torch.uint8, device=x_shard.device)
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    fn = lib().coc_allgather_matmul_trans_w if trans_w else lib().coc_allgather_matmul
    _check(fn(
        _ptr(x_shard), _peer_array(peers, rank), _ptr(w), _ptr(y), _ptr(gathered_out) if v2 else None,
        world, rank, m, n, k, _dtype_code(x_shard), split, int(bool(deterministic)),
        _ptr(ws) if not v2 else None, ws_bytes, _stream(stream, x_shard.device)))
    return (y, gathered_out) if v2 else y


def allgather_matmul_noalloc(x_shard, peers, w, rank, *, y=None, split=4, deterministic=False, stream=None):
    """ALL_GATHER_MATMUL through the allocation-free entry point: the gathered
    matrix and the counters live in the library's static device array
    (m x k x element size <= 64 MiB).  Returns y."""
    world = len(peers)
    shard, k = x_shard.shape
    m = shard * world
    n = w.shape[1]
    y = _empty((m, n), x_shard) if y is None else y
    _check(lib().coc_allgather_matmul_noalloc(
        _ptr(x_shard), _peer_array(peers, rank), _ptr(w), _ptr(y), world, rank, m, n, k, _dtype_code(x_shard),
        split, int(bool(deterministic)), _stream(stream, x_shard.device)))
    return y


def weight_grad(g, dy, *, dw=None, stream=None):
    """dW = G^T @ dY (k x n) for G m x k (e.g. V2's gathered matrix) and dY m x n."""
    m, k = g.shape
    n = dy.shape[1]
    dw = _empty((k, n), g) if dw is None else dw
    _check(lib().coc_weight_grad(_ptr(g), _ptr(dy), _ptr(dw), m, n, k, _dtype_code(g),
                                 _stream(stream, g.device)))
    return dw


def _counts_array(counts):
    """(ctypes int64 array, (split, world, experts), total rows) of a
    split x world x experts nested sequence or array of row counts."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(counts, dtype=np.int64))
    if c.ndim != 3:
        raise ValueError(f"counts must be split x world x experts, got shape {c.shape}")
    arr = (_i64 * c.size)(*c.ravel().tolist())
    return arr, c.shape, int(c.sum())


def alltoall_grouped_matmul(x_own, peers, counts, w, rank, *, y=None, recv_out=None, stream=None):
    """MoE dispatch all-to-all, then the experts' grouped matmul.

    counts[p][r][e]: rows source r routes to local expert e in sequence piece p.
    x_own / peers[r]: the rows this rank / source r sends here (piece, then
    expert order); w: experts x k x n.  Returns (y, recv): recv the received
    rows (piece, expert, source order), y[j] = recv[j] @ w[expert of j]."""
    arr, (split, world, experts), total = _counts_array(counts)
    k, n = w.shape[1], w.shape[2]
    y = _empty((total, n), w) if y is None else y
    recv_out = _empty((total, k), w) if recv_out is None else recv_out
    _check(lib().coc_alltoall_grouped_matmul(
        _ptr(x_own), _peer_array(peers, rank), arr, _ptr(w), _ptr(y), _ptr(recv_out), world, rank, experts,
        n, k, _dtype_code(w), split, _stream(stream, w.device)))
    return y, recv_out


def grouped_matmul_alltoall(h, w, counts, rank, *, peer_out=None, y_own=None, y_local=None, stream=None):
    """The experts' grouped matmul, then the MoE combine all-to-all.

    h: the received rows (piece, expert, source order), total x k; w: experts
    x k x n.  Every row of y_local = h @ w[expert] goes back to its source:
    y_own receives this rank's rows, peer_out[r] source r's.  Returns
    (y_own, peer_out, y_local)."""
    import numpy as np
    arr, (split, world, experts), total = _counts_array(counts)
    k, n = w.shape[1], w.shape[2]
    rows = np.asarray(counts, dtype=np.int64).sum(axis=(0, 2))
    y_local = _empty((total, n), w) if y_local is None else y_local
    y_own = _empty((int(rows[rank]), n), w) if y_own is None else y_own
    if peer_out is None:
        peer_out = [None if r == rank else _empty((int(rows[r]), n), w) for r in range(world)]
    _check(lib().coc_grouped_matmul_alltoall(
        _ptr(h), _ptr(w), _ptr(y_local), _ptr(y_own), _peer_array(peer_out, rank), arr, world, rank, experts,
        n, k, _dtype_code(w), split, _stream(stream, w.device)))
    return y_own, peer_out, y_local


def matmul_all_reduce_w8a16(x, w_q, scales, mode, peers, rank, *, group_size=128, y=None,
                            partial_out=None, split=4, deterministic=False, stream=None):
    """w8A16 MATMUL_ALL_REDUCE (fp16 x, int8 w_q, fp16 scales).  Returns (y, partial_out)."""
    import torch
    if x.dtype != torch.float16 or scales.dtype != torch.float16 or w_q.dtype != torch.int8:
        raise TypeError("w8a16 takes fp16 x, int8 w_q and fp16 scales")
    m, k = x.shape
    n = w_q.shape[1]
    code = QUANT_MODES[mode] if isinstance(mode, str) else int(mode)
    y = _empty((m, n), x) if y is None else y
    partial_out = _empty((m, n), x) if partial_out is None else partial_out
    _check(lib().coc_matmul_all_reduce_w8a16(
        _ptr(x), _ptr(w_q), _ptr(scales), code, group_size, _ptr(y), _ptr(partial_out),
        _peer_array(peers, rank), len(peers), rank, m, n, k, split, int(bool(deterministic)),
        None, 0, _stream(stream, x.device)))
    return y, partial_out


def check_waits(stream=None, device=None) -> None:
    """Raise CocError(COC_ERR_TIMEOUT) if a hand-over wait of the library's work
    on `stream` (default: the current stream) gave up since the last check."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    _check(lib().coc_check_waits(s.cuda_stream))


def workspace_bytes(op: int, m: int, n: int, k: int, dt: int, world: int, split: int) -> int:
    return int(lib().coc_workspace_bytes(op, m, n, k, dt, world, split))


def plan(op: int, m: int, world: int, rank: int, split: int):
    """Chunk descriptors of a pipeline (host only, no GPU needed)."""
    buf = (Chunk * 8)()
    nch = _i32(0)
    _check(lib().coc_plan(op, m, world, rank, split, buf, 8, ctypes.byref(nch)))
    return [{f: getattr(buf[i], f) for f, _ in Chunk._fields_} for i in range(nch.value)]


def profile_enable(on: bool) -> None:
    lib().coc_profile_enable(1 if on else 0)


def profile_stamps(buf) -> None:
    """Point the kernels' activity records at `buf`, a zeroed int64 device
    tensor of 3 x records words (coc.h describes the records); None turns them off."""
    if buf is None:
        lib().coc_profile_stamps(None, 0)
    else:
        lib().coc_profile_stamps(buf.data_ptr(), buf.numel() // 3)


def profile_stamp_count() -> int:
    """Records handed out to launches since the buffer was set."""
    return int(lib().coc_profile_stamp_count())


def diag_mfma_loop(operands, out, workgroups: int, iters: int, stream=None) -> float:
    """Enqueue the MFMA-rate diagnostic (coc.h, coc_diag_mfma_loop) on the
    current stream: `operands` a bf16 device tensor, `out` a float32 device
    tensor of at least workgroups x 256 elements.  Returns the launch's flops."""
    import torch
    assert operands.is_cuda and out.is_cuda and out.dtype == torch.float32
    s = _stream(stream, operands.device)
    _check(lib().coc_diag_mfma_loop(operands.data_ptr(), operands.numel() * operands.element_size(),
                                     out.data_ptr(), out.numel(), workgroups, iters, s))
    return float(workgroups) * 4 * iters * 8 * 32768


def profile_read():
    """Per kernel class: (total ms, launches, algorithmic work) since the last read."""
    ms = (ctypes.c_double * 3)()
    cnt = (_i64 * 3)()
    work = (ctypes.c_double * 3)()
    _check(lib().coc_profile_read(ms, cnt, work))
    return {KCLASS[i]: {"ms": ms[i], "launches": cnt[i], "work": work[i]} for i in range(3)}


def profile_records(max_records: int = 1 << 16):
    """Per-launch (class, start ms, end ms, work) records since the last read."""
    cls = (_i32 * max_records)()
    t0 = (ctypes.c_double * max_records)()
    t1 = (ctypes.c_double * max_records)()
    work = (ctypes.c_double * max_records)()
    n = _i32(0)
    _check(lib().coc_profile_records(cls, t0, t1, work, max_records, ctypes.byref(n)))
    return [(KCLASS[cls[i]], t0[i], t1[i], work[i]) for i in range(min(n.value, max_records))]
