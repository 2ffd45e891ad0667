"""Statistics of the seeded workload generators (CPU only)."""

import numpy as np
import pytest

from synth import configs, dense, graphs
from synth.graphs import CSR


def _sorted_unique(csr: CSR) -> bool:
    k = csr.row_of_edge() * csr.n_cols + csr.col_idx.astype(np.int64)
    return bool(np.all(np.diff(k) > 0))


def _valid(csr: CSR):
    rp = csr.row_ptr.astype(np.int64)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == len(csr.col_idx)
    assert csr.col_idx.dtype == np.int32 and csr.row_ptr.dtype == np.int32
    if csr.nnz:
        assert csr.col_idx.min() >= 0 and csr.col_idx.max() < csr.n_cols


def test_c1_and_p4():
    for name, n in (("c1", 2048), ("p4", 384)):
        c = configs.make_config(name)
        csr = c["csr"]
        _valid(csr)
        assert csr.n_rows == n and _sorted_unique(csr)
        assert abs(csr.degrees().mean() - 18) < 1.0
        assert c["V"].shape == (n, 32 if name == "c1" else 64)
        assert c["V"].min() >= -1 and c["V"].max() <= 1
    # deterministic
    a, b = configs.make_config("c1"), configs.make_config("c1")
    assert np.array_equal(a["csr"].col_idx, b["csr"].col_idx) and np.array_equal(a["V"], b["V"])


def test_c5b_window_pattern():
    csr = configs.config_pattern("c5b")
    _valid(csr)
    d = csr.degrees()
    assert csr.n_rows == 16384 and csr.nnz == 10_383_360
    assert (d[:64] == 16384).all() and d[64] == 320 and d.min() == 320 and d[5000] == 576
    assert _sorted_unique(csr)
    r = 5000
    cols = csr.col_idx[csr.row_ptr[r]:csr.row_ptr[r + 1]]
    assert cols.tolist() == list(range(64)) + list(range(r - 256, r + 256))


def test_c4_skew():
    csr = configs.config_pattern("c4")
    _valid(csr)
    d = csr.degrees()
    assert csr.n_rows == 1_000_000 and csr.nnz == 32_000_000
    assert (d == 0).sum() == 300_000
    assert (d == 200_000).sum() == 78
    top = np.sort(d)[::-1]
    assert top[:17].sum() > 0.10 * csr.nnz
    assert _sorted_unique(csr)


def test_c2_powerlaw():
    csr = configs.config_pattern("c2")
    _valid(csr)
    d = csr.degrees()
    assert csr.n_rows == 232_965
    assert abs(csr.nnz - 114.6e6) < 0.001 * 114.6e6
    assert d.max() <= 20_000 and d.max() > 19_000 and np.median(d) == 6
    assert _sorted_unique(csr)


@pytest.mark.slow
def test_c3_symmetric_lognormal():
    import scipy.sparse as sp

    csr = configs.config_pattern("c3")
    _valid(csr)
    d = csr.degrees()
    assert csr.n_rows == 2_449_029
    assert abs(csr.nnz - 123.7e6) < 0.002 * 123.7e6
    assert 15_000 < d.max() <= 17_000 and np.median(d) == 21
    A = sp.csr_matrix((np.ones(csr.nnz, np.int8), csr.col_idx, csr.row_ptr), shape=(csr.n_rows,) * 2)
    assert (A != A.T).nnz == 0 and A.diagonal().sum() == 0
    assert _sorted_unique(csr)


def test_sample_columns_uniform_subsets():
    rng = np.random.default_rng(3)
    deg = np.array([0, 1, 5, 64, 65, 300, 999, 1000])
    col = graphs.sample_columns(deg, 1000, rng)
    csr = CSR(len(deg), 1000, np.concatenate([[0], np.cumsum(deg)]).astype(np.int32), col)
    assert _sorted_unique(csr)
    assert csr.col_idx[csr.row_ptr[-2]:].tolist() == list(range(1000))
    # uniformity: column frequencies over many short rows
    deg = np.full(20000, 10)
    col = graphs.sample_columns(deg, 50, rng)
    freq = np.bincount(col, minlength=50) / len(col)
    assert np.abs(freq - 1 / 50).max() < 0.003


def test_bf16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0], np.float32)])
    ours = dense.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = dense.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_dense_independent_of_threads(monkeypatch):
    a = dense.dense_normal((3, 1 << 21), 42)
    monkeypatch.setattr(dense, "_threads", lambda: 1)
    b = dense.dense_normal((3, 1 << 21), 42)
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
