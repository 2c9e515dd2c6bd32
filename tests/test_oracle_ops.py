"""Pins for oracle/coc.py.

None of these re-types the oracle's own formula.  They check it against:
  * the tensor-parallel identity the ops exist to implement: a RowParallel
    layer split over T ranks along K sums back to the unsplit product
    (all-reduce), or to row blocks of it (reduce-scatter); a ColumnParallel
    layer fed the gathered sequence equals the unsplit product (all-gather);
  * brute force with exact rationals (fractions.Fraction, element loops) on
    tiny non-square inputs, so a transposed operand, a dropped or extra term,
    a wrong slice or a wrong scale index changes the result;
  * identity / one-hot special cases with exact answers;
  * float64 split-K invariance at a moderate size;
  * hand-worked fixed-order sums (tests/golden/fixed_order_sum.txt) and a
    binary32 emulation through the C library's float conversion (struct).
"""
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import coc, formats

GOLDEN_SUM = os.path.join(os.path.dirname(__file__), "golden", "fixed_order_sum.txt")


# ----------------------------------------------------------------- helpers
def dyadic(rng, shape, bits=4, scale_exp=2):
    """Small dyadic values (exact in bf16 and in float64 sums)."""
    return rng.integers(-(1 << bits), (1 << bits) + 1, size=shape).astype(np.float64) / (1 << scale_exp)


def frac_matrix(a):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(a)]


def bf_matmul(A, B):
    m, k, n = len(A), len(B), len(B[0])
    assert len(A[0]) == k
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            s = Fraction(0)
            for l in range(k):
                s += A[i][l] * B[l][j]
            row.append(s)
        out.append(row)
    return out


def to_float(F):
    return np.array([[float(v) for v in row] for row in F])


def tp_row_parallel_case(rng, m, n, kk, T):
    """A RowParallel layer of width T*kk split over T ranks along K."""
    xf = dyadic(rng, (m, T * kk))
    wf = dyadic(rng, (T * kk, n))
    xs = [xf[:, r * kk:(r + 1) * kk] for r in range(T)]
    ws = [wf[r * kk:(r + 1) * kk, :] for r in range(T)]
    full = to_float(bf_matmul(frac_matrix(xf), frac_matrix(wf)))
    shard_products = [to_float(bf_matmul(frac_matrix(xs[r]), frac_matrix(ws[r]))) for r in range(T)]
    return xs, ws, full, shard_products


# ----------------------------------------------------------------- all-reduce
@pytest.mark.parametrize("T,rank", [(1, 0), (2, 0), (2, 1), (3, 2), (4, 1)])
def test_all_reduce_equals_unsplit_layer(T, rank):
    rng = np.random.default_rng(10 + T * 7 + rank)
    m, n, kk = 5, 3, 4
    xs, ws, full, shard_products = tp_row_parallel_case(rng, m, n, kk, T)
    peers = [p.copy() for p in shard_products]
    peers[rank] = np.full((m, n), np.nan)          # own slot must be ignored
    y, p = oracle.matmul_all_reduce(xs[rank], ws[rank], peers, rank)
    assert np.array_equal(y, full)
    assert np.array_equal(p, shard_products[rank])


# ----------------------------------------------------------------- reduce-scatter
@pytest.mark.parametrize("T,rank", [(1, 0), (2, 1), (4, 0), (4, 3)])
def test_reduce_scatter_equals_row_block_of_unsplit_layer(T, rank):
    rng = np.random.default_rng(50 + T * 3 + rank)
    b, n, kk = 2, 3, 5
    m = b * T
    xs, ws, full, shard_products = tp_row_parallel_case(rng, m, n, kk, T)
    peers = [p.copy() for p in shard_products]
    peers[rank] = np.full((m, n), np.nan)
    # rows of peers outside this rank's slice are never part of the result
    for r in range(T):
        if r != rank:
            mask = np.ones(m, bool)
            mask[rank * b:(rank + 1) * b] = False
            peers[r][mask] = np.nan
    y, p = oracle.matmul_reduce_scatter(xs[rank], ws[rank], peers, rank)
    assert y.shape == (b, n)
    assert np.array_equal(y, full[rank * b:(rank + 1) * b])
    assert np.array_equal(p, shard_products[rank])
    # a sampled evaluation returns the same rows
    ys, ps = oracle.matmul_reduce_scatter(xs[rank], ws[rank], peers, rank, rows=[b - 1, 0])
    assert np.array_equal(ys, full[[rank * b + b - 1, rank * b]])


# ----------------------------------------------------------------- all-gather
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_allgather_matmul_equals_unsplit_sequence(T):
    rng = np.random.default_rng(80 + T)
    b, k, n = 2, 4, 3
    xf = dyadic(rng, (b * T, k))
    w = dyadic(rng, (k, n))
    shards = [xf[r * b:(r + 1) * b] for r in range(T)]
    y, g = oracle.allgather_matmul(shards, w)
    assert np.array_equal(g, xf)
    assert np.array_equal(y, to_float(bf_matmul(frac_matrix(xf), frac_matrix(w))))


# ----------------------------------------------------------------- backward pair
def bf_weight_grad(G, D):
    """dW[i][j] = sum over rows t of G[t][i] * D[t][j], element loops (exact)."""
    m, k, n = len(G), len(G[0]), len(D[0])
    out = []
    for i in range(k):
        row = []
        for j in range(n):
            s = Fraction(0)
            for t in range(m):
                s += G[t][i] * D[t][j]
            row.append(s)
        out.append(row)
    return out


@pytest.mark.parametrize("m,k,n", [(1, 1, 1), (5, 3, 2), (7, 4, 6), (3, 6, 5)])
def test_weight_grad_brute_force(m, k, n):
    rng = np.random.default_rng(300 + m * 31 + k * 7 + n)
    g = dyadic(rng, (m, k))
    dy = dyadic(rng, (m, n))
    assert np.array_equal(oracle.weight_grad(g, dy), to_float(bf_weight_grad(frac_matrix(g), frac_matrix(dy))))


def test_weight_grad_identities():
    """One-hot rows of dY pick rows of G (dW[:, j] = G[t, :] where dY[t, j] = 1),
    and the gradient of the gathered sequence is the sum of the shards'."""
    rng = np.random.default_rng(17)
    m, k, n = 6, 4, 3
    g = dyadic(rng, (m, k))
    dy = np.zeros((m, n))
    for j, t in enumerate((4, 0, 2)):
        dy[t, j] = 1.0
    dw = oracle.weight_grad(g, dy)
    for j, t in enumerate((4, 0, 2)):
        assert np.array_equal(dw[:, j], g[t])
    dy = dyadic(rng, (m, n))
    parts = [oracle.weight_grad(g[r * 2:(r + 1) * 2], dy[r * 2:(r + 1) * 2]) for r in range(3)]
    assert np.array_equal(oracle.weight_grad(g, dy), parts[0] + parts[1] + parts[2])
    with pytest.raises(ValueError):
        oracle.weight_grad(g, dy[:5])


# ----------------------------------------------------------------- w8a16
def bf_dequant(q, s, mode, group):
    K, N = q.shape
    out = []
    for kk in range(K):
        row = []
        for nn in range(N):
            if mode == "per_tensor":
                sc = s[0]
            elif mode == "per_channel":
                sc = s[nn]
            else:
                sc = s[kk // group][nn]
            row.append(Fraction(int(q[kk, nn])) * Fraction(float(sc)))
        out.append(row)
    return out


@pytest.mark.parametrize("mode", ["per_tensor", "per_channel", "per_group"])
def test_w8a16_brute_force(mode):
    rng = np.random.default_rng({"per_tensor": 1, "per_channel": 2, "per_group": 3}[mode])
    m, K, N, group, T, rank = 3, 6, 5, 2, 2, 1
    x = dyadic(rng, (m, K))
    q = rng.integers(-127, 128, size=(K, N))
    # fp16 scales with distinct values per channel / group
    if mode == "per_tensor":
        s = formats.round_to(rng.uniform(0.001, 0.02, 1), "f16")
        s_arg = s
        s_bf = list(s)
    elif mode == "per_channel":
        s = formats.round_to(rng.uniform(0.001, 0.02, N), "f16")
        s_arg = s
        s_bf = list(s)
    else:
        s = formats.round_to(rng.uniform(0.001, 0.02, (K // group, N)), "f16")
        s_arg = s
        s_bf = [list(r) for r in s]
    wt = bf_dequant(q, s_bf, mode, group)
    assert np.array_equal(oracle.dequant_weight(q, s_arg, mode, group), to_float(wt))
    peer = dyadic(rng, (m, N))
    peers = [peer, np.full((m, N), np.nan)]
    y, p = oracle.matmul_all_reduce_w8a16(x, q, s_arg, mode, group, peers, rank)
    pf = bf_matmul(frac_matrix(x), wt)
    exact_y = [[pf[i][j] + Fraction(float(peer[i, j])) for j in range(N)] for i in range(m)]
    # float64 holds these sums exactly only up to rounding; compare in Fractions
    for i in range(m):
        for j in range(N):
            assert abs(Fraction(float(p[i, j])) - pf[i][j]) <= abs(pf[i][j]) * Fraction(1, 2 ** 50)
            assert abs(Fraction(float(y[i, j])) - exact_y[i][j]) <= (abs(exact_y[i][j]) + 1) * Fraction(1, 2 ** 50)


def test_dequant_mode_identities():
    rng = np.random.default_rng(7)
    K, N, g = 256, 24, 128
    q = rng.integers(-127, 128, size=(K, N))
    s0 = formats.round_to(np.array([0.0137]), "f16")
    per_t = oracle.dequant_weight(q, s0, "per_tensor")
    per_c = oracle.dequant_weight(q, np.full(N, s0[0]), "per_channel")
    assert np.array_equal(per_t, per_c)
    sc = formats.round_to(rng.uniform(0.001, 0.02, N), "f16")
    per_c2 = oracle.dequant_weight(q, sc, "per_channel")
    per_g = oracle.dequant_weight(q, np.tile(sc, (K // g, 1)), "per_group", g)
    assert np.array_equal(per_c2, per_g)
    # a per-group scale table that changes along K must change the result
    sg = np.tile(sc, (K // g, 1))
    sg[1] *= 2
    assert not np.array_equal(oracle.dequant_weight(q, sg, "per_group", g), per_c2)
    with pytest.raises(ValueError):
        oracle.dequant_weight(q[:100], sg, "per_group", g)


# ----------------------------------------------------------------- special cases
def test_identity_and_one_hot():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 9))
    assert np.array_equal(oracle.matmul(x, np.eye(9)), x)
    w = rng.standard_normal((9, 4))
    idx = rng.integers(0, 9, 7)
    oh = np.zeros((7, 9))
    oh[np.arange(7), idx] = 1.0
    assert np.array_equal(oracle.matmul(oh, w), w[idx])
    with pytest.raises(ValueError):
        oracle.matmul(x, w.T)


def test_split_k_invariance_float64():
    rng = np.random.default_rng(11)
    m, n, T, kk = 64, 48, 8, 96
    xf = rng.standard_normal((m, T * kk))
    wf = rng.standard_normal((T * kk, n)) * 0.02
    peers = [xf[:, r * kk:(r + 1) * kk] @ wf[r * kk:(r + 1) * kk] for r in range(T)]
    for rank in (0, 5):
        y, _ = oracle.matmul_all_reduce(xf[:, rank * kk:(rank + 1) * kk], wf[rank * kk:(rank + 1) * kk], peers, rank)
        ref = xf @ wf
        assert oracle.normwise_rel_error(y, ref) < 1e-12


# ----------------------------------------------------------------- fixed-order sum
def _golden_sums():
    rows = []
    with open(GOLDEN_SUM) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            dt = parts[0]
            vals = []
            for t in parts[1:]:
                if not t.startswith(("0x", "-0x")):
                    break
                vals.append(float.fromhex(t))
            rows.append((dt, vals[:-1], vals[-1]))
    return rows


@pytest.mark.parametrize("dtype,partials,expected", _golden_sums())
def test_fixed_order_sum_golden(dtype, partials, expected):
    got = oracle.reduce_fixed_order([np.array([v]) for v in partials], dtype)
    assert got[0] == expected


def _f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_fixed_order_sum_vs_scalar_binary32(dtype):
    rng = np.random.default_rng(21)
    T, n = 8, 2000
    parts = [formats.round_dtype(rng.standard_normal(n) * (1 + r), dtype) for r in range(T)]
    got = oracle.reduce_fixed_order(parts, dtype)
    exp = np.empty(n)
    for j in range(n):
        acc = _f32(parts[0][j])
        for r in range(1, T):
            acc = _f32(acc + parts[r][j])     # inputs are binary32 values: the double sum is exact
        exp[j] = acc
    exp = formats.round_dtype(exp, dtype)
    assert np.array_equal(got, exp)
    if dtype == "f32":
        # binary32 partials: the order matters, reversing it changes some bits
        rev = oracle.reduce_fixed_order(parts[::-1], "f32")
        assert not np.array_equal(rev, got)


def test_normwise_rel_error():
    ref = np.array([[3.0, 4.0]])
    assert oracle.normwise_rel_error(ref, ref) == 0.0
    assert oracle.normwise_rel_error(ref + np.array([[0.0, 0.5]]), ref) == pytest.approx(0.1)
    assert oracle.normwise_rel_error(np.zeros(2), np.zeros(2)) == 0.0
