"""bf16 operands with fp32 accumulation (BASELINE-stated tolerance 1e-2 for
bf16 inputs): SpMM with bf16 features, SDDMM with bf16 row operands and the
scores-given attention with bf16 node values, under every schedule the
selector can pick, on the skew graph of the fp32 parity tests.  The oracle
reads the same bf16 values exactly (widened to fp32), so the only error left
is the fp32 accumulation's, and the tests also hold it to the fp32 bound."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
import oracle  # noqa: E402
from synth import to_bf16_bits  # noqa: E402
from gpu_util import TOL_BF16, TOL_F32, assert_close, bf16_dev, dev  # noqa: E402
from test_gpu_parity import pattern_dev, sched_id, schedules, skew_graph  # noqa: E402

THREADS = oracle.default_threads()


def bf16_pair(rng, shape):
    """(bit patterns, device bf16 tensor, exact fp32 values) of N(0,1) draws."""
    bits = to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return bits, bf16_dev(bits), oracle.bf16_to_f32(bits)


def close(got, ref, mag, what):
    e = assert_close(got, ref, mag, TOL_BF16, what)
    assert e <= TOL_F32, f"{what}: {e:.2e} (fp32 accumulation of exact bf16 inputs)"
    return e


@pytest.fixture(scope="module")
def skew():
    return skew_graph(1)


@pytest.mark.parametrize("F", [2, 6, 32, 64, 100, 602])
def test_spmm_bf16_every_schedule(skew, F):
    csr = skew
    rng = np.random.default_rng(700 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    _, Xd, Xf = bf16_pair(rng, (csr.n_cols, F))
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, Xf, threads=THREADS)
    rp, ci = pattern_dev(csr)
    v = dev(vals)
    p, _ = csa.make_problem("spmm", rp, ci, v, Xd)
    assert p.dtype == csa._ffi.DTYPE_BF16
    ss = schedules(p)
    assert all(s.vec in (2, 4, 8) and not s.flags for s in ss)
    for s in ss:
        Y = csa.spmm(rp, ci, v, Xd, schedule=s)
        close(Y.cpu().numpy(), ref, mag, sched_id(s))
    close(csa.spmm(rp, ci, v, Xd).cpu().numpy(), ref, mag, "auto")


@pytest.mark.parametrize("K", [2, 8, 64, 128, 602])
def test_sddmm_bf16_every_schedule(K):
    csr = skew_graph(7, n_rows=2000, n_cols=30_000, giant=25_000)
    rng = np.random.default_rng(800 + K)
    _, Ud, Uf = bf16_pair(rng, (csr.n_rows, K))
    _, Vd, Vf = bf16_pair(rng, (csr.n_cols, K))
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, Uf, Vf, threads=THREADS)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("sddmm", rp, ci, Ud, Vd)
    for s in schedules(p):
        out = csa.sddmm(rp, ci, Ud, Vd, schedule=s)
        close(out.cpu().numpy(), ref, mag, sched_id(s))
    close(csa.sddmm(rp, ci, Ud, Vd).cpu().numpy(), ref, mag, "auto")


def test_bf16_strided_views_and_mixed_errors(skew):
    """bf16 column views (leading dimension > width) and row offsets keep the
    widest aligned access they allow; mixed U / V dtypes and odd widths are
    refused on the host."""
    csr = skew
    rng = np.random.default_rng(5)
    bits, Xd, Xf = bf16_pair(rng, (csr.n_cols, 140))
    rp, ci = pattern_dev(csr)
    for a, b in ((0, 128), (4, 132), (2, 100), (6, 140)):
        view = Xd[:, a:b]
        ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, np.ascontiguousarray(Xf[:, a:b]), threads=THREADS)
        p, _ = csa.make_problem("spmm", rp, ci, None, view)
        for s in schedules(p, thorough=False):
            close(csa.spmm(rp, ci, None, view, schedule=s).cpu().numpy(), ref, mag, f"view {a}:{b} {sched_id(s)}")
    U = dev(rng.standard_normal((csr.n_rows, 8)).astype(np.float32))
    with pytest.raises(TypeError):
        csa.sddmm(rp, ci, U, Xd[:, :8])
    with pytest.raises(csa.CsrError):
        csa.spmm(rp, ci, None, Xd[:, :7])        # odd width: CSR_ERR_SHAPE from the library


@pytest.mark.parametrize("F", [8, 64, 602])
def test_format_bf16(skew, F):
    csr = skew
    rng = np.random.default_rng(1000 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    _, Xd, Xf = bf16_pair(rng, (csr.n_cols, F))
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, Xf, threads=THREADS)
    rp, ci = pattern_dev(csr)
    for P, T in ((4, 0), (16, 64)):
        h = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)
        hv = csa.hybrid_values(h, dev(vals))
        p = csa.hybrid_problem(h, "spmm", hv, Xd)
        for s in schedules(p, thorough=False):
            close(csa.hybrid_spmm(h, hv, Xd, schedule=s).cpu().numpy(), ref, mag, f"P{P} {sched_id(s)}")
    _, Ud, Uf = bf16_pair(rng, (csr.n_rows, 8))
    _, Vd, Vf = bf16_pair(rng, (csr.n_cols, 8))
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, Uf, Vf, threads=THREADS)
    h = csa.hybrid_format(rp, ci, csr.n_cols, 8)
    close(csa.hybrid_sddmm(h, Ud, Vd).cpu().numpy(), ref, mag, "format sddmm bf16")
