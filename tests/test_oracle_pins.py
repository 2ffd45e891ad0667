"""Pins of the CPU oracle to facts outside itself.

Each check below follows from the definitions of the operations (AutoSAGE
page, Abstract: CSR SpMM, CSR SDDMM and the attention pipeline SDDMM ->
row-softmax -> SpMM; POPCORNBENCH trace page, task statement and kernels:
softmax over each destination's incoming edge scores, zero output for a
destination with no edge) or from mathematics, and none reuses the oracle's own
code: dense matrix algebra with numpy/scipy, hand-worked values, closed forms
and invariants.
"""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from synth import random_small_graph, to_bf16_bits, bf16_bits_to_f32
from synth.graphs import CSR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_of(csr, vals):
    """Dense matrix of a CSR pattern; duplicate entries add."""
    A = np.zeros((csr.n_rows, csr.n_cols))
    np.add.at(A, (csr.row_of_edge(), csr.col_idx.astype(np.int64)), vals)
    return A


def dense_attention(csr, scores, V, scale=1.0):
    """Softmax attention written over the edge list: one column per stored
    entry, masked rows -> 0, then a dense product."""
    n, nnz = csr.n_rows, csr.nnz
    rows = csr.row_of_edge()
    S = np.full((n, nnz), -np.inf)
    S[rows, np.arange(nnz)] = scale * np.asarray(scores, dtype=np.float64)
    P = np.zeros_like(S)
    live = csr.degrees() > 0
    if live.any():
        P[live] = sp_softmax(S[live], axis=1)
    return P @ np.asarray(V, dtype=np.float64)[csr.col_idx], P[rows, np.arange(nnz)]


def rel_err(a, b, mag):
    mag = np.asarray(mag)
    diff = np.abs(np.asarray(a) - np.asarray(b))
    return float(np.max(diff / np.maximum(mag, 1e-300))) if diff.size else 0.0


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "worked_4node.json")) as f:
        g = json.load(f)
    csr = CSR(4, 4, np.array(g["row_ptr"], np.int32), np.array(g["col_idx"], np.int32))
    return g, csr


def test_golden_spmm(oracle_lib):
    g, csr = _golden()
    X = np.array(g["features"], np.float32)
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, np.array(g["spmm"]["vals"], np.float32), X)
    assert np.array_equal(Y, np.array(g["spmm"]["expected"], float))


def test_golden_sddmm(oracle_lib):
    g, csr = _golden()
    out, _ = oracle.sddmm(csr.row_ptr, csr.col_idx, np.array(g["sddmm"]["U"], np.float32),
                          np.array(g["sddmm"]["V"], np.float32))
    assert np.array_equal(out, np.array(g["sddmm"]["expected"], float))


def test_golden_attention(oracle_lib):
    g, csr = _golden()
    table = {"0": 0.0, "ln 2": np.log(2.0), "ln 3": np.log(3.0)}
    sc = np.array([table.get(s, None) if s in table else float(s) for s in g["attention"]["scores"]],
                  np.float32)
    out, _, p = oracle.attention(csr.row_ptr, csr.col_idx, sc, np.array(g["features"], np.float32),
                                 want_probs=True)
    assert np.max(np.abs(out - np.array(g["attention"]["expected"]))) < 1e-6
    assert np.max(np.abs(p - np.array(g["attention"]["expected_probs"]))) < 1e-6
    assert out[2].tolist() == [0.0, 0.0]


# --------------------------------------------------------------------------
# dense brute force on random small graphs
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_spmm_dense_bruteforce(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    n, m, F = int(rng.integers(1, 60)), int(rng.integers(1, 70)), int(rng.integers(1, 20))
    csr = random_small_graph(n, m, rng.random() * 0.4, rng, empty_frac=0.2, allow_dup=True)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((m, F)).astype(np.float32)
    Y, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X)
    ref = dense_of(csr, vals) @ X.astype(np.float64)
    refmag = dense_of(csr, np.abs(vals)) @ np.abs(X.astype(np.float64))
    assert np.allclose(Y, ref, rtol=0, atol=1e-12 * max(1.0, refmag.max()))
    assert np.allclose(mag, refmag, rtol=1e-13, atol=0)
    # missing values mean a_e = 1
    Y1, _ = oracle.spmm(csr.row_ptr, csr.col_idx, None, X)
    assert np.allclose(Y1, dense_of(csr, np.ones(csr.nnz)) @ X, atol=1e-12 * max(1, np.abs(X).sum()))


@pytest.mark.parametrize("seed", range(12))
def test_sddmm_dense_bruteforce(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    n, m, K = int(rng.integers(1, 60)), int(rng.integers(1, 70)), int(rng.integers(1, 40))
    csr = random_small_graph(n, m, rng.random() * 0.4, rng, empty_frac=0.2, allow_dup=True)
    U = rng.standard_normal((n, K)).astype(np.float32)
    V = rng.standard_normal((m, K)).astype(np.float32)
    out, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V)
    full = U.astype(np.float64) @ V.astype(np.float64).T
    assert np.allclose(out, full[csr.row_of_edge(), csr.col_idx], rtol=0, atol=1e-12 * K)
    fullmag = np.abs(U.astype(np.float64)) @ np.abs(V.astype(np.float64)).T
    assert np.allclose(mag, fullmag[csr.row_of_edge(), csr.col_idx], rtol=1e-13)


@pytest.mark.parametrize("seed", range(12))
def test_attention_dense_bruteforce(oracle_lib, seed):
    rng = np.random.default_rng(200 + seed)
    n, m, F = int(rng.integers(1, 60)), int(rng.integers(1, 70)), int(rng.integers(1, 20))
    csr = random_small_graph(n, m, rng.random() * 0.5, rng, empty_frac=0.25, allow_dup=seed % 2 == 1)
    scores = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((m, F)).astype(np.float32)
    scale = [1.0, 0.125, 2.5][seed % 3]
    out, mag, p = oracle.attention(csr.row_ptr, csr.col_idx, scores, V, scale, want_probs=True)
    ref, refp = dense_attention(csr, scores, V, scale)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)
    assert np.allclose(p, refp, rtol=0, atol=1e-14)


def _bf16(rng, shape):
    return to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("seed", range(6))
def test_mha_dense_bruteforce(oracle_lib, seed):
    rng = np.random.default_rng(300 + seed)
    n, H, D = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 17))
    csr = random_small_graph(n, n, rng.random() * 0.5, rng, empty_frac=0.2)
    Q, K, Vb = _bf16(rng, (n, H, D)), _bf16(rng, (n, H, D)), _bf16(rng, (n, H, D))
    scale = 1.0 / np.sqrt(D)
    out, mag, p = oracle.mha(csr.row_ptr, csr.col_idx, Q, K, Vb, scale, want_probs=True)
    Qf, Kf, Vf = (bf16_bits_to_f32(a).astype(np.float64) for a in (Q, K, Vb))
    for h in range(H):
        S = Qf[:, h, :] @ Kf[:, h, :].T  # dense scores, then sampled on the pattern
        sc = S[csr.row_of_edge(), csr.col_idx]
        ref, refp = dense_attention(csr, sc, Vf[:, h, :], scale)
        assert np.allclose(out[:, h, :], ref, rtol=0, atol=1e-12)
        assert np.allclose(p[:, h], refp, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_attention_qk_dense_bruteforce(oracle_lib, seed):
    """fp32 queries and keys: per head, dense scores Q_h K_h^T sampled on the
    pattern, then the masked dense softmax attention (duplicates included:
    each stored entry is its own term)."""
    rng = np.random.default_rng(340 + seed)
    n, m = int(rng.integers(1, 40)), int(rng.integers(1, 45))
    H, D = int(rng.integers(1, 4)), int(rng.integers(1, 20))
    csr = random_small_graph(n, m, rng.random() * 0.5, rng, empty_frac=0.2, allow_dup=seed % 2 == 1)
    Q = rng.standard_normal((n, H, D)).astype(np.float32)
    K = rng.standard_normal((m, H, D)).astype(np.float32)
    V = rng.standard_normal((m, H, D)).astype(np.float32)
    scale = [1.0, 0.125, 0.7][seed % 3]
    out, mag, p = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q, K, V, scale, want_probs=True)
    for h in range(H):
        S = Q[:, h, :].astype(np.float64) @ K[:, h, :].astype(np.float64).T
        ref, refp = dense_attention(csr, S[csr.row_of_edge(), csr.col_idx], V[:, h, :], scale)
        assert np.allclose(out[:, h, :], ref, rtol=0, atol=1e-12)
        assert np.allclose(p[:, h], refp, rtol=0, atol=1e-13)
        refmag, _ = dense_attention(csr, S[csr.row_of_edge(), csr.col_idx], np.abs(V[:, h, :]), scale)
        assert np.allclose(mag[:, h, :], refmag, rtol=0, atol=1e-12)
    # one head given as 2-D arrays is the same call with H = 1
    o1, _, _ = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q[:, 0], K[:, 0], V[:, 0], scale)
    assert np.array_equal(o1[:, 0], out[:, 0])


def test_attention_qk_identity_and_uniform(oracle_lib):
    """Identity pattern: every row attends only to itself, out = V exactly;
    keys all equal: uniform weights, out = the mean of the neighbours' V."""
    rng = np.random.default_rng(7)
    n, D = 17, 6
    Q = rng.standard_normal((n, 1, D)).astype(np.float32)
    V = rng.standard_normal((n, 1, D)).astype(np.float32)
    eye = CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32))
    out, _, _ = oracle.attention_qk(eye.row_ptr, eye.col_idx, Q, Q, V, 0.3)
    assert np.array_equal(out, V.astype(np.float64))
    csr = random_small_graph(n, n, 0.4, rng, empty_frac=0.2)
    K = np.tile(rng.standard_normal((1, 1, D)).astype(np.float32), (n, 1, 1))
    out, _, _ = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q, K, V, 1.0)
    for i in range(n):
        cols = csr.col_idx[csr.row_ptr[i]:csr.row_ptr[i + 1]]
        want = V[cols, 0].astype(np.float64).mean(axis=0) if len(cols) else np.zeros(D)
        assert np.allclose(out[i, 0], want, rtol=0, atol=1e-14)


def test_bf16_widening_known_patterns():
    """bfloat16 is the high half of an IEEE float32: known bit patterns."""
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x3FC0, 0x4049], np.uint16)
    want = np.array([1.0, -2.0, np.inf, -np.inf, 0.0, -0.0, 2.0 ** -133, 1.5, 3.140625], np.float32)
    got = oracle.bf16_to_f32(bits)
    assert got.dtype == np.float32 and np.array_equal(got, want)
    assert np.signbit(got[5]) and not np.signbit(got[4])


def test_exhaustive_3x3_patterns(oracle_lib):
    """Every one of the 512 patterns of a 3 x 3 matrix."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 4)).astype(np.float32)
    U = rng.standard_normal((3, 4)).astype(np.float32)
    for mask in range(512):
        M = np.array([(mask >> k) & 1 for k in range(9)], bool).reshape(3, 3)
        rows, cols = np.nonzero(M)
        rp = np.zeros(4, np.int32)
        np.cumsum(M.sum(1), out=rp[1:])
        csr = CSR(3, 3, rp, cols.astype(np.int32))
        vals = rng.standard_normal(len(rows)).astype(np.float32)
        sc = rng.standard_normal(len(rows)).astype(np.float32)
        Y, _ = oracle.spmm(rp, csr.col_idx, vals, X)
        assert np.allclose(Y, dense_of(csr, vals) @ X, atol=1e-12)
        out, _ = oracle.sddmm(rp, csr.col_idx, U, X)
        assert np.allclose(out, (U.astype(float) @ X.astype(float).T)[rows, cols], atol=1e-12)
        att, _, _ = oracle.attention(rp, csr.col_idx, sc, X)
        ref, _ = dense_attention(csr, sc, X)
        assert np.allclose(att, ref, atol=1e-13)
        for r in range(3):
            if not M[r].any():
                assert att[r].tolist() == [0.0] * 4 and Y[r].tolist() == [0.0] * 4


# --------------------------------------------------------------------------
# special cases and closed forms
# --------------------------------------------------------------------------

def _full_pattern(n, m):
    rp = (np.arange(n + 1) * m).astype(np.int32)
    return CSR(n, m, rp, np.tile(np.arange(m, dtype=np.int32), n))


def test_full_pattern_is_dense_softmax_attention(oracle_lib):
    rng = np.random.default_rng(11)
    n, m, F = 17, 23, 9
    csr = _full_pattern(n, m)
    S = rng.standard_normal((n, m)).astype(np.float32)
    V = rng.standard_normal((m, F)).astype(np.float32)
    out, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, S.ravel(), V, scale=0.5)
    ref = sp_softmax(0.5 * S.astype(np.float64), axis=1) @ V.astype(np.float64)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, S.ravel(), V)
    assert np.allclose(Y, S.astype(np.float64) @ V.astype(np.float64), atol=1e-12)


def test_identity_pattern_exact(oracle_lib):
    rng = np.random.default_rng(12)
    n, F = 50, 7
    csr = CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32))
    V = rng.standard_normal((n, F)).astype(np.float32)
    sc = rng.standard_normal(n).astype(np.float32) * 30
    out, _, p = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, want_probs=True)
    assert np.array_equal(out, V.astype(np.float64))
    assert np.array_equal(p, np.ones(n))
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, None, V)
    assert np.array_equal(Y, V.astype(np.float64))


def test_empty_rows_are_positive_zero(oracle_lib):
    rng = np.random.default_rng(13)
    csr = random_small_graph(40, 40, 0.2, rng, empty_frac=0.5)
    V = rng.standard_normal((40, 5)).astype(np.float32)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    out, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V)
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, sc, V)
    empty = csr.degrees() == 0
    assert empty.any()
    for arr in (out, mag, Y):
        assert np.all(arr[empty] == 0) and not np.signbit(arr[empty]).any()


def test_uniform_scores_give_neighbour_mean(oracle_lib):
    rng = np.random.default_rng(14)
    csr = random_small_graph(60, 80, 0.15, rng, empty_frac=0.1)
    V = rng.standard_normal((80, 6)).astype(np.float32)
    sc = np.repeat(rng.standard_normal(60).astype(np.float32) * 5, csr.degrees())
    out, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V)
    for i in range(60):
        cols = csr.col_idx[csr.row_ptr[i]:csr.row_ptr[i + 1]]
        want = V[cols].astype(np.float64).mean(0) if len(cols) else np.zeros(6)
        assert np.allclose(out[i], want, atol=1e-14)


def test_constant_values(oracle_lib):
    rng = np.random.default_rng(15)
    csr = random_small_graph(60, 80, 0.2, rng, empty_frac=0.1)
    c = np.float32(-1.75)
    V = np.full((80, 3), c, np.float32)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    out, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V)
    live = csr.degrees() > 0
    assert np.allclose(out[live], c, atol=1e-14)
    # mean aggregation (values 1/deg) of a constant feature gives the constant
    inv = np.repeat(1.0 / np.maximum(csr.degrees(), 1), csr.degrees())
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, inv.astype(np.float32), V)
    assert np.allclose(Y[live], c, rtol=1e-6)


def test_softmax_rows_sum_to_one(oracle_lib):
    rng = np.random.default_rng(16)
    csr = random_small_graph(100, 100, 0.3, rng, empty_frac=0.1)
    sc = (10 * rng.standard_normal(csr.nnz)).astype(np.float32)
    _, _, p = oracle.attention(csr.row_ptr, csr.col_idx, sc, np.ones((100, 1), np.float32),
                               want_probs=True)
    sums = np.add.reduceat(p, csr.row_ptr[:-1][csr.degrees() > 0])
    assert np.allclose(sums, 1.0, rtol=0, atol=1e-15 * 100)
    assert (p > 0).all() and (p <= 1).all()


def test_shift_invariance_and_overflow(oracle_lib):
    """Adding a constant to every score of a row leaves its output unchanged;
    with a shift of 1000 the exponentials would overflow without subtracting
    the row maximum.  Scores are multiples of 2^-10 so the shifted fp32 values
    are exact."""
    rng = np.random.default_rng(17)
    csr = random_small_graph(50, 60, 0.3, rng, empty_frac=0.1)
    base = (np.round(rng.standard_normal(csr.nnz) * 1024) / 1024).astype(np.float32)
    V = rng.standard_normal((60, 4)).astype(np.float32)
    shift = np.repeat(rng.choice([-1000.0, 80.0, 0.0, 1000.0], 50), csr.degrees()).astype(np.float32)
    a, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, base, V)
    b, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, base + shift, V)
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)


def test_hard_attention_limit(oracle_lib):
    rng = np.random.default_rng(18)
    csr = random_small_graph(60, 60, 0.3, rng, empty_frac=0.0)
    V = rng.standard_normal((60, 5)).astype(np.float32)
    # a unique maximum per row, at least 0.05 above every other score
    sc = np.empty(csr.nnz, np.float32)
    for i in range(60):
        b, e = csr.row_ptr[i], csr.row_ptr[i + 1]
        k = e - b
        if k:
            s = rng.permutation(k).astype(np.float32) * 0.05
            sc[b:e] = s
    out, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, scale=1000.0)
    for i in range(60):
        b, e = csr.row_ptr[i], csr.row_ptr[i + 1]
        if e > b:
            j = csr.col_idx[b + int(np.argmax(sc[b:e]))]
            assert np.allclose(out[i], V[j], atol=1e-6)


def test_spmm_linearity(oracle_lib):
    rng = np.random.default_rng(19)
    csr = random_small_graph(40, 50, 0.3, rng)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.integers(-8, 8, (50, 6)).astype(np.float32)
    Z = rng.integers(-8, 8, (50, 6)).astype(np.float32)
    a, b = 3.0, -0.5  # small integers and halves keep every sum exact-ish
    lhs, _ = oracle.spmm(csr.row_ptr, csr.col_idx, vals, (a * X + b * Z).astype(np.float32))
    rx, _ = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X)
    rz, _ = oracle.spmm(csr.row_ptr, csr.col_idx, vals, Z)
    assert np.allclose(lhs, a * rx + b * rz, atol=1e-12)


def test_sddmm_spmm_duality(oracle_lib):
    """sum_e <U_row(e), V_col(e)> = sum_i <U_i, (A1 V)_i>, A1 the 0/1 pattern."""
    rng = np.random.default_rng(20)
    csr = random_small_graph(45, 55, 0.3, rng, empty_frac=0.1)
    U = rng.standard_normal((45, 8)).astype(np.float32)
    V = rng.standard_normal((55, 8)).astype(np.float32)
    out, _ = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V)
    Y, _ = oracle.spmm(csr.row_ptr, csr.col_idx, None, V)
    assert np.isclose(out.sum(), np.sum(U.astype(np.float64) * Y), rtol=1e-12)


def test_relabeling_equivariance(oracle_lib):
    rng = np.random.default_rng(21)
    n = 50
    csr = random_small_graph(n, n, 0.2, rng, empty_frac=0.1)
    V = rng.standard_normal((n, 4)).astype(np.float32)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    perm = rng.permutation(n)  # new id of old node i is perm[i]
    inv = np.argsort(perm)
    rows = csr.row_of_edge()
    new_rows, new_cols = perm[rows], perm[csr.col_idx]
    order = np.lexsort((new_cols, new_rows))
    rp = np.zeros(n + 1, np.int32)
    np.cumsum(np.bincount(new_rows, minlength=n), out=rp[1:])
    V2 = V[inv]
    out, _, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V)
    out2, _, _ = oracle.attention(rp, new_cols[order].astype(np.int32), sc[order], V2)
    assert np.allclose(out2[perm], out, atol=1e-14)


def test_thread_count_does_not_change_results(oracle_lib):
    rng = np.random.default_rng(22)
    csr = random_small_graph(300, 200, 0.1, rng, empty_frac=0.2)
    V = rng.standard_normal((200, 5)).astype(np.float32)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    a = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, threads=1)[0]
    b = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, threads=7)[0]
    assert np.array_equal(a, b)
    c = oracle.spmm(csr.row_ptr, csr.col_idx, sc, V, r0=100, r1=250, threads=3)[0]
    assert np.array_equal(c, oracle.spmm(csr.row_ptr, csr.col_idx, sc, V)[0][100:250])


# --------------------------------------------------------------------------
# integer bookkeeping
# --------------------------------------------------------------------------

def test_fnv1a64_published_vectors():
    assert oracle.fnv1a64(b"") == 0xCBF29CE484222325
    assert oracle.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert oracle.fnv1a64(b"foobar") == 0x85944171F73967E8


@pytest.mark.parametrize("seed", range(8))
def test_degree_histogram_bruteforce(seed):
    rng = np.random.default_rng(400 + seed)
    deg = rng.integers(0, 3000, size=500) * (rng.random(500) < 0.8)
    deg[:4] = [0, 1, 2**11, 2**11 - 1]
    rp = np.zeros(501, np.int64)
    np.cumsum(deg, out=rp[1:])
    counts, sums, mx = oracle.degree_histogram(rp)
    c2, s2 = [0] * 33, [0] * 33
    for d in deg.tolist():
        b = int(d).bit_length()  # 0 for d = 0, else floor(log2 d) + 1
        c2[b] += 1
        s2[b] += int(d)
    assert counts.tolist() == c2 and sums.tolist() == s2 and mx == int(deg.max())


@pytest.mark.parametrize("seed", range(10))
def test_merge_path_counting_equals_walk(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(0, 60))
    deg = rng.integers(0, 12, size=n) * (rng.random(n) < 0.7)
    rp = np.zeros(n + 1, np.int32)
    np.cumsum(deg, out=rp[1:])
    for D in (1, 2, 3, 7, 16, 64, 1000):
        x, y = oracle.merge_path_partition(rp, D)
        bx, by = oracle.merge_path_bruteforce(rp, D)
        assert x.tolist() == bx.tolist() and y.tolist() == by.tolist()
        # every chunk holds exactly D items except the last
        items = (x[1:] + y[1:]) - (x[:-1] + y[:-1])
        assert (items[:-1] == D).all() and 0 <= items[-1] <= D


# --------------------------------------------------------------------------
# backward operations: finite differences of the (pinned) forward, closed
# forms, invariants, dense algebra
# --------------------------------------------------------------------------

def _grid_scores(rng, n, lim=2.0):
    """Scores on a 2^-8 grid in [-lim, lim]: s +- 2^-10 is exact in fp32, so a
    central difference perturbs exactly one score by exactly h."""
    return (np.round(rng.uniform(-lim, lim, n) * 256) / 256).astype(np.float32)


@pytest.mark.parametrize("seed", range(4))
def test_softmax_backward_finite_differences(oracle_lib, seed):
    rng = np.random.default_rng(700 + seed)
    csr = random_small_graph(9, 11, 0.4, rng, empty_frac=0.2, allow_dup=True)
    scale = [1.0, 0.5, 0.125, 2.0][seed]
    s = _grid_scores(rng, csr.nnz)
    g = rng.standard_normal(csr.nnz).astype(np.float32)
    zero = np.zeros((csr.n_cols, 1), np.float32)

    def loss(sv):
        p = oracle_lib.attention(csr.row_ptr, csr.col_idx, sv, zero, scale, want_probs=True)[2]
        return float(np.dot(g.astype(np.float64), p))

    p32 = oracle_lib.attention(csr.row_ptr, csr.col_idx, s, zero, scale, want_probs=True)[2].astype(np.float32)
    ds, mag = oracle_lib.softmax_backward(csr.row_ptr, p32, g, scale)
    h = 2.0 ** -10
    fd = np.empty(csr.nnz)
    for e in range(csr.nnz):
        sp, sm = s.copy(), s.copy()
        sp[e] += np.float32(h)
        sm[e] -= np.float32(h)
        fd[e] = (loss(sp) - loss(sm)) / (2 * h)
    assert rel_err(ds, fd, mag) < 1e-4


def test_softmax_backward_two_entry_closed_form(oracle_lib):
    # p1 = logistic(t1 - t2): dL/ds1 = scale p1 p2 (g1 - g2) = -dL/ds2
    rp = np.array([0, 2], np.int32)
    for t1, t2, g1, g2, scale in ((0.5, -1.0, 2.0, -0.5, 1.0), (3.0, 3.0, 1.0, 4.0, 0.25), (-2.0, 1.5, 0.0, 1.0, 2.0)):
        p1 = 1.0 / (1.0 + np.exp(-scale * (t1 - t2)))
        p = np.array([p1, 1 - p1], np.float32)
        ds, _ = oracle_lib.softmax_backward(rp, p, np.array([g1, g2], np.float32), scale)
        want = scale * float(p[0]) * float(p[1]) * (g1 - g2)
        assert abs(ds[0] - want) < 1e-6 and abs(ds[1] + want) < 1e-6


def test_softmax_backward_invariants(oracle_lib):
    rng = np.random.default_rng(710)
    csr = random_small_graph(40, 30, 0.3, rng, empty_frac=0.2)
    zero = np.zeros((csr.n_cols, 1), np.float32)
    p = oracle_lib.attention(csr.row_ptr, csr.col_idx, rng.standard_normal(csr.nnz).astype(np.float32), zero,
                             1.0, want_probs=True)[2].astype(np.float32)
    g = rng.standard_normal(csr.nnz).astype(np.float32)
    ds, _ = oracle_lib.softmax_backward(csr.row_ptr, p, g, 0.7)
    live = csr.degrees() > 0
    starts = csr.row_ptr[:-1][live]
    # over each row the gradient sums to scale * S * (1 - sum p): zero for an
    # exact softmax, here the rounding of p to fp32
    S = np.add.reduceat(p.astype(np.float64) * g, starts)
    psum = np.add.reduceat(p.astype(np.float64), starts)
    assert np.max(np.abs(np.add.reduceat(ds, starts) - 0.7 * S * (1 - psum))) < 1e-12
    assert np.max(np.abs(1 - psum)) < 1e-6
    # a gradient constant over a row has no effect beyond that rounding:
    # ds_e = scale * p_e * c_i * (1 - sum p)
    crow = rng.standard_normal(csr.n_rows)
    c = np.repeat(crow, csr.degrees()).astype(np.float32)
    dc, _ = oracle_lib.softmax_backward(csr.row_ptr, p, c, 0.7)
    psum_all = np.bincount(csr.row_of_edge(), weights=p.astype(np.float64), minlength=csr.n_rows)
    left = np.repeat(1 - psum_all, csr.degrees())
    assert np.max(np.abs(dc - 0.7 * p * c.astype(np.float64) * left)) < 1e-12
    assert np.max(np.abs(dc)) < 1e-6


@pytest.mark.parametrize("seed", range(3))
def test_attention_backward_finite_differences(oracle_lib, seed):
    rng = np.random.default_rng(720 + seed)
    csr = random_small_graph(8, 10, 0.45, rng, empty_frac=0.2, allow_dup=seed == 2)
    F, scale = 3, [1.0, 0.125, 0.5][seed]
    s = _grid_scores(rng, csr.nnz)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)

    def loss(sv):
        out = oracle_lib.attention(csr.row_ptr, csr.col_idx, sv, V, scale)[0]
        return float(np.sum(dO.astype(np.float64) * out))

    ds, mag = oracle_lib.attention_backward_scores(csr.row_ptr, csr.col_idx, s, V, dO, scale)
    h = 2.0 ** -10
    fd = np.empty(csr.nnz)
    for e in range(csr.nnz):
        sp, sm = s.copy(), s.copy()
        sp[e] += np.float32(h)
        sm[e] -= np.float32(h)
        fd[e] = (loss(sp) - loss(sm)) / (2 * h)
    assert rel_err(ds, fd, mag) < 1e-4


@pytest.mark.parametrize("seed", range(6))
def test_spmm_transpose_dense(oracle_lib, seed):
    rng = np.random.default_rng(730 + seed)
    csr = random_small_graph(25, 18, 0.2, rng, empty_frac=0.2, allow_dup=seed % 2 == 1)
    vals = rng.standard_normal(csr.nnz)
    dY = rng.standard_normal((csr.n_rows, 4)).astype(np.float32)
    dX, mag = oracle_lib.spmm_transpose(csr.row_ptr, csr.col_idx, vals, dY, csr.n_cols)
    want = dense_of(csr, vals).T @ dY.astype(np.float64)
    assert rel_err(dX, want, mag) < 1e-12
    ones, _ = oracle_lib.spmm_transpose(csr.row_ptr, csr.col_idx, None, dY, csr.n_cols)
    assert np.allclose(ones, dense_of(csr, np.ones(csr.nnz)).T @ dY.astype(np.float64), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_transpose_definition(seed):
    rng = np.random.default_rng(740 + seed)
    csr = random_small_graph(30, 23, 0.15, rng, empty_frac=0.3, allow_dup=seed % 2 == 1)
    t_rp, t_ci, perm = oracle.transpose(csr.row_ptr, csr.col_idx, csr.n_cols)
    assert sorted(perm.tolist()) == list(range(csr.nnz))
    At = CSR(csr.n_cols, csr.n_rows, t_rp, t_ci)
    vals = rng.standard_normal(csr.nnz)
    assert np.array_equal(dense_of(At, vals[perm]), dense_of(csr, vals).T)
    # each column lists its rows in increasing order, ties in entry order
    for j in range(csr.n_cols):
        seg = perm[t_rp[j]:t_rp[j + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(csr.col_idx[seg] == j)
    # transposing twice gives back the pattern with each row's entries ordered
    # by (column, original position): the original order when it was sorted
    rp2, ci2, perm2 = oracle.transpose(t_rp, t_ci, csr.n_rows)
    order = np.lexsort((np.arange(csr.nnz), csr.col_idx, csr.row_of_edge()))
    assert np.array_equal(rp2, csr.row_ptr) and np.array_equal(ci2, csr.col_idx[order])
    assert np.array_equal(perm[perm2], order)


# ---------------------------------------------------------------------------
# column-part segment format
# ---------------------------------------------------------------------------

def test_hybrid_format_hand_example():
    """Worked by hand from the definition: 10 columns in 4 parts of 3 columns
    (0-2, 3-5, 6-8, 9); row 0 lists unsorted columns, row 1 is empty."""
    row_ptr = [0, 5, 5, 7, 10]
    col_idx = [5, 0, 9, 3, 1,  # row 0: parts 1 0 3 1 0
               7, 8,           # row 2: parts 2 2
               2, 6, 4]        # row 3: parts 0 2 1
    want = {
        "part_cols": 3,
        # segments (part, row): (0,0) = e1 e4; (0,3) = e7; (1,0) = e0 e3; (1,3) = e9;
        # (2,2) = e5 e6; (2,3) = e8; (3,0) = e2
        "perm": [1, 4, 7, 0, 3, 9, 5, 6, 8, 2],
        "col_idx": [0, 1, 2, 5, 3, 4, 7, 8, 6, 9],
        "seg_ptr": [0, 2, 3, 5, 6, 8, 9, 10],
        "seg_row": [0, 3, 0, 3, 2, 3, 0],
        "seg_part": [0, 0, 1, 1, 2, 2, 3],
        "row_seg_ptr": [0, 3, 3, 4, 7],
        "row_seg": [0, 2, 6, 4, 1, 3, 5],
    }
    for build in (oracle.hybrid_format_loops, oracle.hybrid_format):
        got = build(row_ptr, col_idx, 10, 4)
        for k, v in want.items():
            assert np.array_equal(np.asarray(got[k]), np.asarray(v)), (build.__name__, k)
    # rows with fewer than 3 entries kept whole (row 2): one segment in part 4, after all column parts
    want_whole = {
        "perm": [1, 4, 7, 0, 3, 9, 8, 2, 5, 6],
        "col_idx": [0, 1, 2, 5, 3, 4, 6, 9, 7, 8],
        "seg_ptr": [0, 2, 3, 5, 6, 7, 8, 10],
        "seg_row": [0, 3, 0, 3, 3, 0, 2],
        "seg_part": [0, 0, 1, 1, 2, 3, 4],
        "row_seg_ptr": [0, 3, 3, 4, 7],
        "row_seg": [0, 2, 5, 6, 1, 3, 4],
    }
    for build in (oracle.hybrid_format_loops, oracle.hybrid_format):
        got = build(row_ptr, col_idx, 10, 4, whole_below=3)
        for k, v in want_whole.items():
            assert np.array_equal(np.asarray(got[k]), np.asarray(v)), (build.__name__, "whole", k)
    # one part: the segments are the non-empty rows, in order
    one = oracle.hybrid_format(row_ptr, col_idx, 10, 1)
    assert one["perm"].tolist() == list(range(10)) and one["seg_row"].tolist() == [0, 2, 3]
    assert one["seg_ptr"].tolist() == [0, 5, 7, 10] and one["row_seg_ptr"].tolist() == [0, 1, 1, 2, 3]


@pytest.mark.parametrize("seed", range(8))
def test_hybrid_format_bruteforce(seed):
    """The stable-sort construction equals the loop construction on small
    patterns: unsorted and duplicate columns, empty rows, fewer columns than
    parts, no entries."""
    rng = np.random.default_rng(760 + seed)
    n_cols = [1, 3, 7, 20, 33, 64, 5, 40][seed]
    csr = random_small_graph(25, n_cols, 0.0 if seed == 6 else 0.3, rng, empty_frac=0.2, allow_dup=seed % 2 == 1)
    for P in (1, 2, 4, 8, 16, 32, 64, 256):
        for T in (0, 4, 1000):
            a = oracle.hybrid_format_loops(csr.row_ptr, csr.col_idx, n_cols, P, whole_below=T)
            b = oracle.hybrid_format(csr.row_ptr, csr.col_idx, n_cols, P, whole_below=T)
            for k in a:
                assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), (P, T, k)


@pytest.mark.parametrize("seed", range(4))
def test_hybrid_format_invariants(seed):
    rng = np.random.default_rng(770 + seed)
    csr = random_small_graph(300, 500, 0.05, rng, empty_frac=0.2, allow_dup=seed % 2 == 1)
    rows = csr.row_of_edge()
    deg = np.diff(csr.row_ptr)
    for P, T in ((2, 0), (8, 0), (32, 0), (8, 25), (32, 30)):
        h = oracle.hybrid_format(csr.row_ptr, csr.col_idx, csr.n_cols, P, whole_below=T)
        perm, sp, sr, spart = h["perm"], h["seg_ptr"], h["seg_row"], h["seg_part"]
        assert h["part_cols"] == -(-500 // P)
        assert sorted(perm.tolist()) == list(range(csr.nnz))  # a permutation of the entries
        assert np.array_equal(h["col_idx"], csr.col_idx[perm])
        assert sp[0] == 0 and sp[-1] == csr.nnz and np.all(np.diff(sp) > 0)  # no empty segment
        whole = deg < T
        for s in range(len(sr)):
            seg = perm[sp[s]:sp[s + 1]]
            assert np.all(rows[seg] == sr[s]) and np.all(np.diff(seg) > 0)  # one row, original order
            if whole[sr[s]]:  # a row kept whole: all its entries, in part P
                assert spart[s] == P and len(seg) == deg[sr[s]]
            else:
                assert np.all(csr.col_idx[seg] // h["part_cols"] == spart[s])
        key = spart * csr.n_rows + sr
        assert np.all(np.diff(key) > 0)  # ordered by (part, row), each pair once
        # every row's entries are its segments, by part
        for r in range(csr.n_rows):
            mine = h["row_seg"][h["row_seg_ptr"][r]:h["row_seg_ptr"][r + 1]]
            assert np.all(sr[mine] == r) and np.all(np.diff(spart[mine]) > 0)
            got = np.concatenate([perm[sp[s]:sp[s + 1]] for s in mine]) if len(mine) else np.zeros(0, int)
            e = np.arange(csr.row_ptr[r], csr.row_ptr[r + 1])
            want = e if whole[r] else e[np.argsort(csr.col_idx[e] // h["part_cols"], kind="stable")]
            assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(4))
def test_hybrid_product_identity(oracle_lib, seed):
    """The product summed segment by segment (each row's segments in part
    order) is the dense product: the format only re-associates the sum."""
    rng = np.random.default_rng(780 + seed)
    csr = random_small_graph(40, 60, 0.2, rng, empty_frac=0.2, allow_dup=seed % 2 == 1)
    vals = rng.standard_normal(csr.nnz).astype(np.float32).astype(np.float64)  # the oracle reads fp32 values
    X = rng.standard_normal((60, 5)).astype(np.float32)
    h = oracle.hybrid_format(csr.row_ptr, csr.col_idx, 60, 4, whole_below=(0, 6, 12, 100)[seed])
    ref, mag = oracle_lib.spmm(csr.row_ptr, csr.col_idx, vals, X)
    part_rows = np.zeros((len(h["seg_row"]), 5))
    for s in range(len(h["seg_row"])):
        for k in range(h["seg_ptr"][s], h["seg_ptr"][s + 1]):
            part_rows[s] += vals[h["perm"][k]] * X[h["col_idx"][k]].astype(np.float64)
    Y = np.zeros((csr.n_rows, 5))
    for r in range(csr.n_rows):
        for s in h["row_seg"][h["row_seg_ptr"][r]:h["row_seg_ptr"][r + 1]]:
            Y[r] += part_rows[s]
    assert rel_err(Y, ref, mag) < 1e-12
    assert rel_err(Y, dense_of(csr, vals) @ X.astype(np.float64), mag) < 1e-12


def test_gpu_error_measure_fails_on_nan():
    # the parity tests' error measure: a NaN anywhere is an infinite error,
    # so aggregating blocks with max() cannot pass over it
    import gpu_util

    ref = np.array([1.0, 2.0, 3.0])
    mag = np.array([1.0, 2.0, 3.0])
    assert gpu_util.max_err(np.array([1.0, np.nan, 3.0]), ref, mag) == float("inf")
    assert max(0.0, gpu_util.max_err(np.array([np.nan, 2.0, 3.0]), ref, mag)) == float("inf")
    with pytest.raises(AssertionError):
        gpu_util.max_err(np.array([np.nan]), np.array([0.0]), np.array([0.0]))  # zero magnitude must be exactly 0
    assert gpu_util.max_err(ref, ref, mag) == 0.0


@pytest.mark.parametrize("seed", range(3))
def test_attention_qk_backward_composition_finite_differences(oracle_lib, seed):
    """The gradients of the attention from queries and keys as the library
    composes them, written with oracle functions: s = SDDMM(Q, K), d s from
    the scores-given backward, dQ = A_ds K and dK = A_ds^T Q; against
    central differences of the oracle's forward in every entry of Q and K."""
    rng = np.random.default_rng(740 + seed)
    csr = random_small_graph(7, 8, 0.45, rng, empty_frac=0.15, allow_dup=seed == 2)
    D, F, scale = 3, 3, [0.5, 1.0, 0.25][seed]
    grid = lambda shape: (np.round(rng.uniform(-1.5, 1.5, shape) * 256) / 256).astype(np.float32)  # noqa: E731
    Q, K = grid((csr.n_rows, D)), grid((csr.n_cols, D))
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)

    def loss(q, k):
        out = oracle_lib.attention_qk(csr.row_ptr, csr.col_idx, q, k, V, scale)[0]
        return float(np.sum(dO.astype(np.float64) * out[:, 0, :]))

    s, _ = oracle_lib.sddmm(csr.row_ptr, csr.col_idx, Q, K)
    ds, mag_ds = oracle_lib.attention_backward_scores(csr.row_ptr, csr.col_idx, s.astype(np.float32), V, dO, scale)
    dQ, _ = oracle_lib.spmm(csr.row_ptr, csr.col_idx, ds, K)
    magQ, _ = oracle_lib.spmm(csr.row_ptr, csr.col_idx, mag_ds, np.abs(K))
    dK, _ = oracle_lib.spmm_transpose(csr.row_ptr, csr.col_idx, ds, Q, csr.n_cols)
    magK, _ = oracle_lib.spmm_transpose(csr.row_ptr, csr.col_idx, mag_ds, np.abs(Q), csr.n_cols)
    h = 2.0 ** -10
    for M, G, mag, which in ((Q, dQ, magQ, 0), (K, dK, magK, 1)):
        fd = np.empty(M.shape)
        for idx in np.ndindex(M.shape):
            mp, mm = M.copy(), M.copy()
            mp[idx] += np.float32(h)
            mm[idx] -= np.float32(h)
            lp = loss(mp, K) if which == 0 else loss(Q, mp)
            lm = loss(mm, K) if which == 0 else loss(Q, mm)
            fd[idx] = (lp - lm) / (2 * h)
        assert rel_err(G, fd, mag + 1e-30) < 1e-4, which
