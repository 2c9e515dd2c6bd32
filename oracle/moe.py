"""Plain fp64 definitions of the MoE expert all-to-all + grouped matmul pair, one
expert-parallel rank's share.

Test infrastructure only (see oracle/__init__.py).

Pages cited (by title, section):
  * Ampipe page -- MindSpeed feature page "Ampipe流水通信隐藏": "Problem analysis"
    (an all-to-all before and one after the expert MLP exchange tokens between
    the ranks of the expert-parallel group, serial with the compute) and
    "Solution" / "Approach" (the input is cut along the sequence into
    independent pieces whose communication and compute are then pipelined).
  * Overlap blog -- "MindSpeed LLM通信计算重叠与MC2如何榨干昇腾芯片算力", second
    layer (EP MC2: the expert all-to-all fused with the experts' grouped matmul
    into one pipeline).

Readings (the pages give no layouts):
  * ``counts[p][r][e]`` rows: in sequence piece p, source rank r routes that
    many token rows to local expert e of this rank.  The pieces are the
    sequence pieces of the Ampipe split (the first index is the degree).
  * Source rank r's rows for this rank are ordered piece-major, then by local
    expert, then in r's own order: ``sends[r]`` (this rank's own rows at
    index ``rank``).
  * The received matrix orders rows piece-major, then by local expert, then
    by source rank, then in the source's order, so that every (piece, expert)
    group is one contiguous block of rows for the grouped matmul.
  * The grouped matmul multiplies each row by its expert's weight ``ws[e]``
    (k x n).  The combine returns every row of the grouped matmul's output to
    the rank it came from, at the position it had in that rank's rows.
  * Values are those of the storage dtype passed as float64; products of two
    such values are exact in float64 (see oracle/coc.py).
"""
from __future__ import annotations

import numpy as np


def _counts(counts) -> np.ndarray:
    c = np.asarray(counts, dtype=np.int64)
    if c.ndim != 3 or (c < 0).any():
        raise ValueError(f"counts must be a [pieces][world][experts] array of row counts >= 0, got {c.shape}")
    return c


def _blocks_of_source(c: np.ndarray, r: int):
    """(piece, expert) -> (first row, rows) in source r's rows for this rank."""
    out = {}
    row = 0
    for p in range(c.shape[0]):
        for e in range(c.shape[2]):
            out[(p, e)] = (row, int(c[p, r, e]))
            row += int(c[p, r, e])
    return out, row


def received_order(counts):
    """The received rows as a list of (piece, expert, source, index within the
    source's block), in the received matrix's row order."""
    c = _counts(counts)
    order = []
    for p in range(c.shape[0]):
        for e in range(c.shape[2]):
            for r in range(c.shape[1]):
                order.extend((p, e, r, i) for i in range(int(c[p, r, e])))
    return order


def alltoall_dispatch(sends, counts) -> np.ndarray:
    """The dispatch all-to-all (Ampipe page, "Problem analysis": the exchange
    before the expert MLP): every source's rows for this rank, regrouped into
    the received order.  A pure permutation of rows."""
    c = _counts(counts)
    world = c.shape[1]
    if len(sends) != world:
        raise ValueError(f"{len(sends)} send blocks for world {world}")
    blocks = []
    for r in range(world):
        b, total = _blocks_of_source(c, r)
        s = np.asarray(sends[r], dtype=np.float64)
        if s.shape[0] != total:
            raise ValueError(f"source {r} sends {s.shape[0]} rows, counts say {total}")
        blocks.append((b, s))
    rows = []
    for p in range(c.shape[0]):
        for e in range(c.shape[2]):
            for r in range(world):
                b, s = blocks[r]
                r0, n = b[(p, e)]
                rows.append(s[r0:r0 + n])
    k = np.asarray(sends[0]).shape[1] if world else 0
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, k))


def group_rows(counts):
    """(piece, expert) -> (first row, rows) in the received order."""
    c = _counts(counts)
    out = {}
    row = 0
    for p in range(c.shape[0]):
        for e in range(c.shape[2]):
            n = int(c[p, :, e].sum())
            out[(p, e)] = (row, n)
            row += n
    return out


def grouped_matmul(h, counts, ws) -> np.ndarray:
    """The experts' grouped matmul (Overlap blog, EP MC2's GroupedMatMul): each
    (piece, expert) block of the received rows times that expert's k x n
    weight, in float64."""
    h = np.asarray(h, dtype=np.float64)
    ws = [np.asarray(w, dtype=np.float64) for w in ws]
    c = _counts(counts)
    if len(ws) != c.shape[2]:
        raise ValueError(f"{len(ws)} expert weights for {c.shape[2]} experts")
    n = ws[0].shape[1]
    y = np.zeros((h.shape[0], n))
    for (p, e), (r0, rows) in group_rows(c).items():
        if h.shape[1] != ws[e].shape[0]:
            raise ValueError(f"rows of width {h.shape[1]} times a {ws[e].shape} weight")
        y[r0:r0 + rows] = h[r0:r0 + rows] @ ws[e]
    return y


def alltoall_grouped_matmul(sends, counts, ws):
    """Dispatch all-to-all, then the experts' first matmul.  Returns (Y, R):
    R the received rows (the all-to-all's output), Y = each row of R times its
    expert's weight."""
    recv = alltoall_dispatch(sends, counts)
    return grouped_matmul(recv, counts, ws), recv


def alltoall_combine(y, counts):
    """The combine all-to-all (Ampipe page, "Problem analysis": the exchange
    after the expert MLP): row j of the received order goes back to its source
    rank at the position it had there.  Returns one block per source rank."""
    y = np.asarray(y, dtype=np.float64)
    c = _counts(counts)
    world = c.shape[1]
    outs = []
    for r in range(world):
        _, total = _blocks_of_source(c, r)
        outs.append(np.zeros((total, y.shape[1])))
    pos = [_blocks_of_source(c, r)[0] for r in range(world)]
    row = 0
    for p in range(c.shape[0]):
        for e in range(c.shape[2]):
            for r in range(world):
                r0, n = pos[r][(p, e)]
                outs[r][r0:r0 + n] = y[row:row + n]
                row += n
    if row != y.shape[0]:
        raise ValueError(f"{y.shape[0]} rows, counts say {row}")
    return outs


def grouped_matmul_alltoall(h, counts, ws):
    """The experts' second matmul, then the combine all-to-all.  Returns
    (outs, Y): outs[r] the rows going back to rank r (this rank's own at index
    ``rank``), Y the grouped matmul's output in the received order."""
    y = grouped_matmul(h, counts, ws)
    return alltoall_combine(y, counts), y
