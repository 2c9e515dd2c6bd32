"""Pins of the MoE all-to-all + grouped matmul oracle (oracle/moe.py) against
things other than itself: a plain sort of tagged rows (the received layout),
scaled-identity experts (which expert each row meets), exact integer
arithmetic token by token, the reduction to one plain matmul, the dispatch /
combine round trip, and the invariance of each token's result under the
sequence split.  No page prints a worked example for these ops."""
import itertools

import numpy as np
import pytest

import oracle


def _tagged_sends(counts, k=6):
    """Send blocks whose rows carry their tag (piece, expert, source, index) in
    the first four columns, built in each source's documented order."""
    c = np.asarray(counts)
    P, W, E = c.shape
    sends, tags = [], []
    for r in range(W):
        rows, t = [], []
        for p in range(P):
            for e in range(E):
                for i in range(c[p, r, e]):
                    rows.append([p, e, r, i] + [0] * (k - 4))
                    t.append((p, e, r, i))
        sends.append(np.array(rows, dtype=np.float64).reshape(len(rows), k))
        tags.append(t)
    return sends, tags


COUNTS = [
    [[2, 0, 3], [1, 4, 0]],          # 1 piece, 2 sources, 3 experts (zeros included)
    [[[1, 2], [0, 1], [3, 0]],
     [[2, 2], [1, 0], [0, 1]]],      # 2 pieces, 3 sources, 2 experts
]


@pytest.mark.parametrize("counts", [np.array(COUNTS[0])[None], np.array(COUNTS[1])])
def test_received_layout_is_sorted_tags(counts):
    """The received rows are the union of all sent rows in lexicographic
    (piece, expert, source, index) order."""
    sends, tags = _tagged_sends(counts)
    recv = oracle.alltoall_dispatch(sends, counts)
    want = sorted(itertools.chain(*tags))
    got = [tuple(int(v) for v in row[:4]) for row in recv]
    assert got == want
    assert oracle.received_order(counts) == want


def test_each_row_meets_its_expert():
    """Expert e's weight is (e + 2) * I: every output row is its input row
    times the factor of the expert in its tag."""
    counts = np.array(COUNTS[1])
    sends, _ = _tagged_sends(counts, k=8)
    ws = [(e + 2) * np.eye(8) for e in range(counts.shape[2])]
    y, recv = oracle.alltoall_grouped_matmul(sends, counts, ws)
    for row_in, row_out in zip(recv, y):
        e = int(row_in[1])
        assert np.array_equal(row_out, (e + 2) * row_in)


def test_exact_integers_token_by_token():
    """Small integer inputs: every token's result, computed alone with Python
    integers, equals its row of the dispatch output (found by tag) and its
    place in the combine output."""
    rng = np.random.default_rng(3)
    counts = np.array(COUNTS[1])
    P, W, E = counts.shape
    k, n = 5, 4
    sends = [rng.integers(-9, 10, size=(int(counts[:, r, :].sum()), k)).astype(np.float64) for r in range(W)]
    ws = [rng.integers(-9, 10, size=(k, n)).astype(np.float64) for _ in range(E)]
    y, recv = oracle.alltoall_grouped_matmul(sends, counts, ws)
    outs, _ = oracle.grouped_matmul_alltoall(recv, counts, ws)
    order = oracle.received_order(counts)
    for r in range(W):
        row = 0
        for p in range(P):
            for e in range(E):
                for i in range(counts[p, r, e]):
                    x = [int(v) for v in sends[r][row]]
                    want = [sum(x[kk] * int(ws[e][kk][j]) for kk in range(k)) for j in range(n)]
                    j = order.index((p, e, r, i))
                    assert [int(v) for v in y[j]] == want
                    assert [int(v) for v in recv[j]] == x
                    assert [int(v) for v in outs[r][row]] == want
                    row += 1


def test_one_piece_one_expert_is_a_plain_matmul():
    """With one piece and one expert the received matrix is the sources' rows
    stacked in rank order, and the product is one ordinary matmul."""
    rng = np.random.default_rng(4)
    counts = np.array([[[3], [0], [5]]])
    sends = [rng.standard_normal((int(c), 7)) for c in counts[0, :, 0]]
    w = rng.standard_normal((7, 6))
    y, recv = oracle.alltoall_grouped_matmul(sends, counts, [w])
    assert np.array_equal(recv, np.vstack(sends))
    np.testing.assert_allclose(y, np.vstack(sends) @ w, rtol=1e-13, atol=1e-13)


def test_combine_undoes_dispatch():
    """With identity experts, combining the dispatched rows returns every
    source's rows unchanged, in place."""
    rng = np.random.default_rng(5)
    for counts in (np.array(COUNTS[0])[None], np.array(COUNTS[1]), np.zeros((2, 2, 3), dtype=np.int64)):
        W, E = counts.shape[1], counts.shape[2]
        sends = [rng.standard_normal((int(counts[:, r, :].sum()), 5)) for r in range(W)]
        ws = [np.eye(5)] * E
        y, recv = oracle.alltoall_grouped_matmul(sends, counts, ws)
        outs, _ = oracle.grouped_matmul_alltoall(recv, counts, ws)
        for r in range(W):
            assert outs[r].shape == sends[r].shape
            assert np.array_equal(outs[r], sends[r])


def test_sequence_split_moves_rows_only():
    """Cutting each source's tokens into two sequence pieces changes where a
    token's row sits, not its result: per token the outputs agree exactly."""
    rng = np.random.default_rng(6)
    W, E, T, k, n = 3, 2, 10, 6, 5
    expert = rng.integers(0, E, size=(W, T))          # one routed row per token
    x = rng.integers(-5, 6, size=(W, T, k)).astype(np.float64)
    ws = [rng.integers(-5, 6, size=(k, n)).astype(np.float64) for _ in range(E)]

    def run(pieces):
        bounds = np.linspace(0, T, pieces + 1).astype(int)
        counts = np.zeros((pieces, W, E), dtype=np.int64)
        sends, ids = [], []
        for r in range(W):
            rows, tok = [], []
            for p in range(pieces):
                for e in range(E):
                    for t in range(bounds[p], bounds[p + 1]):
                        if expert[r, t] == e:
                            rows.append(x[r, t])
                            tok.append(t)
                            counts[p, r, e] += 1
            sends.append(np.array(rows).reshape(len(rows), k))
            ids.append(tok)
        outs, _ = oracle.grouped_matmul_alltoall(oracle.alltoall_dispatch(sends, counts), counts, ws)
        return {(r, t): tuple(outs[r][i]) for r in range(W) for i, t in enumerate(ids[r])}

    one, two = run(1), run(2)
    assert one == two
    for (r, t), v in one.items():
        assert np.array_equal(np.array(v), x[r, t] @ ws[expert[r, t]])


def test_bad_inputs_raise():
    with pytest.raises(ValueError):
        oracle.alltoall_dispatch([np.zeros((1, 4))], np.array([[[-1]]]))
    with pytest.raises(ValueError):
        oracle.alltoall_dispatch([np.zeros((2, 4))], np.array([[[1]]]))
    with pytest.raises(ValueError):
        oracle.grouped_matmul(np.zeros((1, 4)), np.array([[[1, 0]]]), [np.zeros((4, 3))])
