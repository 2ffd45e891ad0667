"""The Python binding's host-side checks and its workspace handling.

Every wrong shape, count or dtype is rejected on the host with ValueError or
TypeError before any kernel is launched; workspaces are per (device, stream),
a caller may pass its own, and a buffer a captured graph refers to stays
valid when a later call needs a larger one."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
from csr_sparse_attention_amd import ops  # noqa: E402
from synth import graphs  # noqa: E402
from gpu_util import dev  # noqa: E402


@pytest.fixture(scope="module")
def g():
    rng = np.random.default_rng(11)
    csr = graphs.random_small_graph(300, 200, 0.05, rng)
    return csr, dev(csr.row_ptr), dev(csr.col_idx)


def f32(*shape):
    return torch.randn(*shape, device="cuda")


def no_launch(fn):
    """Runs fn, which must raise ValueError or TypeError from the host-side
    checks, before it enqueues anything."""
    torch.cuda.synchronize()
    with pytest.raises((ValueError, TypeError)):
        fn()
    torch.cuda.synchronize()


def test_spmm_rejects_bad_shapes(g):
    csr, rp, ci = g
    n, m, nnz = csr.n_rows, csr.n_cols, csr.nnz
    X = f32(m, 16)
    vals = f32(nnz)
    no_launch(lambda: csa.spmm(rp, ci, vals, X, out=f32(n - 1, 16)))       # too few output rows
    no_launch(lambda: csa.spmm(rp, ci, vals, X, out=f32(n, 15)))           # wrong width
    no_launch(lambda: csa.spmm(rp, ci, vals, X, out=torch.empty((n, 16), dtype=torch.float64, device="cuda")))
    no_launch(lambda: csa.spmm(rp, ci, f32(nnz - 1), X))                   # one value short
    no_launch(lambda: csa.spmm(rp, ci, vals, f32(m)))                      # 1-D X
    no_launch(lambda: csa.spmm(rp, ci, vals, X.cpu()))                     # X on the host
    no_launch(lambda: csa.spmm(rp.long(), ci, vals, X))                    # int64 row_ptr


def test_sddmm_attention_mha_reject_bad_shapes(g):
    csr, rp, ci = g
    n, m, nnz = csr.n_rows, csr.n_cols, csr.nnz
    no_launch(lambda: csa.sddmm(rp, ci, f32(n - 1, 8), f32(m, 8)))          # U short of rows
    no_launch(lambda: csa.sddmm(rp, ci, f32(n, 8), f32(m, 4)))              # widths differ
    no_launch(lambda: csa.sddmm(rp, ci, f32(n, 8), f32(m, 8), out=f32(nnz - 1)))
    no_launch(lambda: csa.attention(rp, ci, f32(nnz + 1), f32(m, 8)))       # scores of another pattern
    no_launch(lambda: csa.attention(rp, ci, f32(nnz), f32(m, 8), out=f32(n, 9)))
    bf = lambda *s: torch.randn(*s, device="cuda").to(torch.bfloat16)  # noqa: E731
    no_launch(lambda: csa.mha_attention(rp, ci, bf(n - 1, 2, 8), bf(m, 2, 8), bf(m, 2, 8)))
    no_launch(lambda: csa.mha_attention(rp, ci, bf(n, 2, 8), bf(m, 2, 8), bf(m, 2, 8),
                                        out=torch.empty((n, 2, 8), dtype=torch.bfloat16, device="cuda")))
    no_launch(lambda: csa.mha_attention(rp, ci, bf(n, 2, 8), bf(m, 2, 8), bf(m, 2, 8), out=f32(n, 16)))


def test_softmax_gather_hybrid_reject_bad_shapes(g):
    csr, rp, ci = g
    n, m, nnz = csr.n_rows, csr.n_cols, csr.nnz
    s = f32(nnz)
    no_launch(lambda: csa.row_softmax(rp, s, out=f32(nnz - 1)))
    no_launch(lambda: csa.row_softmax_backward(rp, s, f32(nnz - 1)))
    no_launch(lambda: csa.row_softmax_backward(rp, s, s, out=f32(nnz + 1)))
    t = csa.transpose(rp, ci, m)
    no_launch(lambda: csa.gather_values(t.perm, f32(nnz - 1)))
    no_launch(lambda: csa.gather_values(t.perm, s, out=f32(nnz - 1)))
    h = csa.hybrid_format(rp, ci, m, 4)
    no_launch(lambda: csa.hybrid_spmm(h, None, f32(m - 1, 8)))              # X of another column count
    no_launch(lambda: csa.hybrid_spmm(h, None, f32(m, 8), out=f32(n - 1, 8)))
    no_launch(lambda: csa.hybrid_sddmm(h, f32(n - 1, 8), f32(m, 8)))
    no_launch(lambda: csa.hybrid_sddmm(h, f32(n, 8), f32(m, 8), out=f32(nnz - 1)))


def test_caller_workspace_and_per_stream_buffers(g):
    csr, rp, ci = g
    X = f32(csr.n_cols, 32)
    ref = csa.spmm(rp, ci, None, X)
    p, _ = csa.make_problem("spmm", rp, ci, None, X)
    need = csa.workspace_size(p)
    mine = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    assert torch.equal(csa.spmm(rp, ci, None, X, workspace=mine), ref)
    no_launch(lambda: csa.spmm(rp, ci, None, X, workspace=mine[: need // 2]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        y = csa.spmm(rp, ci, None, X)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    dev_i = torch.cuda.current_device()
    keys = {k for k in ops._workspaces if k[0] == dev_i}
    assert (dev_i, side.cuda_stream) in keys and (dev_i, torch.cuda.current_stream().cuda_stream) in keys


def test_graph_replays_after_the_workspace_grew(g):
    """A captured call keeps the workspace address it was captured with; a
    later eager call on the same stream that needs a larger workspace must
    not free that buffer, or the replays would write into reused memory."""
    csr, rp, ci = g
    X = f32(csr.n_cols, 8)
    s, _ = csa.select("spmm", rp, ci, None, X)
    out = torch.empty((csr.n_rows, 8), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        csa.spmm(rp, ci, None, X, out=out, schedule=s)
        ref = out.clone()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            csa.spmm(rp, ci, None, X, out=out, schedule=s)
        held = ops._workspaces[(torch.cuda.current_device(), side.cuda_stream)]
        held_ptr = held.data_ptr()
        # a much larger call on the same stream grows the stream's workspace
        big = graphs.csr_from_degrees(np.full(20_000, 60), 20_000, np.random.default_rng(2))
        brp, bci = dev(big.row_ptr), dev(big.col_idx)
        Xb = f32(big.n_cols, 512)
        for k in range(3):
            out.fill_(float("nan"))
            csa.spmm(brp, bci, None, Xb)          # eager work that needs the larger buffer
            junk = torch.full((1 << 22,), 7.0, device="cuda")  # allocations that could reuse freed memory
            gr.replay()
            side.synchronize()
            assert torch.equal(out, ref), k
            del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert any(t.data_ptr() == held_ptr for t in ops._graph_held)
