"""rocSPARSE's outputs against the oracle, before any timing comparison is
quoted: its CSR SpMM (every algorithm bench.py times) over every row of the
power-law workload at F = 32, and its SDDMM over sampled rows of the
log-normal workload at K = 128.  rocSPARSE is a measured comparison beside
this library, never part of its path; skipped where the library is absent."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402,F401
import oracle  # noqa: E402
from synth import configs  # noqa: E402
from gpu_util import TOL_F32, compare_all_rows, dev, max_err  # noqa: E402

THREADS = min(16, oracle.default_threads())


def _rocsparse():
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    try:
        return bench.Rocsparse(torch, reps=1)
    except OSError:
        pytest.skip("librocsparse not available")


@pytest.mark.timeout(900)
def test_rocsparse_spmm_matches_oracle_c2():
    rs = _rocsparse()
    csr = configs.config_pattern("c2")
    F = 32
    vals = configs.config_dense("c2", "vals", csr)
    X = configs.config_dense("c2", "X", csr, F)
    rp, ci, vd, Xd = dev(csr.row_ptr), dev(csr.col_idx), dev(vals), dev(X)
    outs = {}
    for name, alg in rs.ALGS.items():
        Y = torch.full((csr.n_rows, F), float("nan"), device="cuda")
        ms, rc = rs.spmm(rp, ci, vd, Xd, Y, alg)
        assert ms is not None, (name, rc)
        outs[name] = Y.cpu().numpy()
    rs.close()
    worst = {n: 0.0 for n in outs}

    def block(r0, r1):
        ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, r0, r1, threads=THREADS)
        for n, Y in outs.items():
            worst[n] = max(worst[n], max_err(Y[r0:r1], ref, mag))
        return ref, mag

    compare_all_rows(outs["default"], block, csr.row_ptr, F, TOL_F32, "rocsparse default")
    print("rocSPARSE SpMM c2 F=32, max error per algorithm:", {n: f"{e:.2e}" for n, e in worst.items()})
    for n, e in worst.items():
        assert e <= TOL_F32, (n, e)


@pytest.mark.timeout(900)
def test_rocsparse_sddmm_matches_oracle_c3():
    rs = _rocsparse()
    csr = configs.config_pattern("c3")
    U = configs.config_dense("c3", "U", csr, 128)
    V = configs.config_dense("c3", "V", csr, 128)
    rp, ci = dev(csr.row_ptr), dev(csr.col_idx)
    # zeros, not NaN: rocSPARSE's SDDMM forms beta * C even for beta = 0
    out = torch.zeros(csr.nnz, device="cuda")
    ms, rc = rs.sddmm(rp, ci, dev(U), dev(V), out)
    rs.close()
    assert ms is not None, rc
    got = out.cpu().numpy()
    rng = np.random.default_rng(3)
    deg = csr.degrees()
    rows = np.unique(np.concatenate([np.argsort(deg)[::-1][:24], rng.choice(csr.n_rows, 400, replace=False)]))
    rp64 = csr.row_ptr.astype(np.int64)
    worst = 0.0
    for r in rows:
        ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, int(r), int(r) + 1)
        worst = max(worst, max_err(got[rp64[r]:rp64[r + 1]], ref, mag))
    print(f"rocSPARSE SDDMM c3 K=128: max error {worst:.2e} over {len(rows)} rows")
    assert worst <= TOL_F32
