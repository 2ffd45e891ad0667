"""The allocation-free SpMM entry point (csr_spmm_noalloc) against csr_spmm
through the C ABI: the same schedule runs the same kernels, so the outputs
must be bit for bit equal, on two calls in a row (the second smaller, the
scratch array keeping the first call's contents), for merge-path schedules
(which keep their partition and split-row pieces in the scratch array) and
row-group schedules; oversized problems are refused before any launch."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
import oracle  # noqa: E402
from synth import graphs  # noqa: E402
from gpu_util import TOL_F32, assert_close, dev  # noqa: E402

_ffi = csa._ffi


def skewed(seed, n_rows, n_cols, giant):
    rng = np.random.default_rng(seed)
    deg = rng.integers(0, 40, n_rows)
    deg[rng.integers(0, n_rows)] = giant
    return graphs.csr_from_degrees(deg, n_cols, rng), rng


def raw_noalloc(ctx, rp, ci, vals, X, Y, sched):
    lib = csa.load_library()
    return lib.csr_spmm_noalloc(ctx.handle, rp.numel() - 1, X.shape[0], ci.numel(), rp.data_ptr(), ci.data_ptr(),
                                None if vals is None else vals.data_ptr(), X.data_ptr(), _ffi.DTYPE_F32, X.shape[1],
                                X.stride(0), Y.data_ptr(), Y.stride(0), ctypes.byref(sched),
                                torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("mapping", ["mergepath", "rowgroup", "segscan"])
def test_noalloc_matches_spmm_twice(mapping):
    ctx = csa.default_context()
    cases = [skewed(1, 6000, 40_000, 30_000) + (64,), skewed(2, 1500, 8000, 6000) + (64,)]
    if mapping == "segscan":
        cases = [(c, r, 4) for c, r, _ in cases]
    for k, (csr, rng, F) in enumerate(cases):  # the second call is smaller than the first
        rp, ci = dev(csr.row_ptr), dev(csr.col_idx)
        vals = rng.standard_normal(csr.nnz).astype(np.float32)
        X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
        vd, Xd = dev(vals), dev(X)
        p, _ = csa.make_problem("spmm", rp, ci, vd, Xd)
        s = csa.default_schedule(p)
        if mapping == "rowgroup":
            s.mapping, s.chunk_items, s.long_row = _ffi.MAP_ROWGROUP, 0, 0
        elif mapping == "segscan":
            s.mapping, s.group_lanes, s.chunk_items, s.long_row = _ffi.MAP_SEGSCAN, 1, 256, 0
            s.passes = 1
        need = csa.workspace_size(p, s)
        assert need <= _ffi.NOALLOC_SCRATCH_BYTES
        ref = csa.spmm(rp, ci, vd, Xd, schedule=s)
        Y = torch.full_like(ref, float("nan"))
        assert raw_noalloc(ctx, rp, ci, vd, Xd, Y, s) == 0, csa.load_library().csr_last_error(ctx.handle)
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), (mapping, k)
        Y2 = csa.spmm_noalloc(rp, ci, vd, Xd, schedule=s)
        assert torch.equal(Y2, ref), (mapping, k)
        want, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=oracle.default_threads())
        assert_close(Y.cpu().numpy(), want, mag, TOL_F32, f"noalloc {mapping} call {k}")


def test_noalloc_refuses_oversized_and_missing_schedule():
    ctx = csa.default_context()
    csr, rng = skewed(3, 50_000, 60_000, 50_000)
    rp, ci = dev(csr.row_ptr), dev(csr.col_idx)
    X = dev(rng.standard_normal((csr.n_cols, 1024)).astype(np.float32))
    p, _ = csa.make_problem("spmm", rp, ci, None, X)
    s = csa.default_schedule(p)
    s.chunk_items = 256
    assert csa.workspace_size(p, s) > _ffi.NOALLOC_SCRATCH_BYTES
    Y = torch.full((csr.n_rows, 1024), 7.0, device="cuda")
    assert raw_noalloc(ctx, rp, ci, None, X, Y, s) == -5
    lib = csa.load_library()
    assert b"scratch" in lib.csr_last_error(ctx.handle)
    assert lib.csr_spmm_noalloc(ctx.handle, csr.n_rows, csr.n_cols, csr.nnz, rp.data_ptr(), ci.data_ptr(), None,
                                X.data_ptr(), 0, 1024, 1024, Y.data_ptr(), 1024, None,
                                torch.cuda.current_stream().cuda_stream) == -1
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())  # nothing was written
