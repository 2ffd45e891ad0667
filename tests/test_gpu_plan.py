"""Planned products (csr_plan_*): the library chooses the layout (plain CSR or
the column-part segment format at some part count and whole-row threshold)
and the product's schedule together, by its cost model and micro-probes,
caches the joint choice and replays it.  Every plan's product is checked
against the oracle; replay is bit-exact; the cache log carries the choice
across contexts."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
import oracle  # noqa: E402
from synth import graphs, to_bf16_bits  # noqa: E402
from gpu_util import TOL_BF16, TOL_F32, assert_close, bf16_dev, dev  # noqa: E402
from test_gpu_parity import pattern_dev, skew_graph  # noqa: E402

THREADS = oracle.default_threads()
_ffi = csa._ffi


def powerlaw_graph(seed, n=60_000, kmax=6000):
    """Columns uniform over 60,000 nodes, heavy-tailed degrees: a gathered
    operand of 15 MB at F = 64, where the format's part counts are candidates."""
    rng = np.random.default_rng(seed)
    deg = graphs.powerlaw_degrees(n, 1.35, kmax)
    return graphs.csr_from_degrees(rng.permutation(deg), n, rng), rng


@pytest.fixture(scope="module")
def pl_graph():
    return powerlaw_graph(5)


@pytest.mark.parametrize("F", [8, 64, 200])
def test_plan_spmm(pl_graph, F):
    csr, rng = pl_graph
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    rp, ci = pattern_dev(csr)
    vd, Xd = dev(vals), dev(X)
    ctx = csa.Context(0, None)
    pl = csa.plan("spmm", rp, ci, vd, Xd, ctx=ctx)
    Y = csa.plan_spmm(pl, Xd, ctx=ctx)
    e = assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, f"plan F={F}")
    print(f"plan spmm F={F}: {pl} max err {e:.2e}")
    # the same input again: the cached choice, replayed bit for bit
    pl2 = csa.plan("spmm", rp, ci, vd, Xd, ctx=ctx)
    assert pl2.choice() == pl.choice() and pl2.signature == pl.signature and pl2.desc.probe_ms == 0.0
    assert torch.equal(csa.plan_spmm(pl2, Xd, ctx=ctx), Y)
    assert torch.equal(csa.plan_spmm(pl, Xd, ctx=ctx), Y)
    # this call's own values, then the plan's again
    v2 = rng.standard_normal(csr.nnz).astype(np.float32)
    ref2, mag2 = oracle.spmm(csr.row_ptr, csr.col_idx, v2, X, threads=THREADS)
    assert_close(csa.plan_spmm(pl, Xd, vals=dev(v2), ctx=ctx).cpu().numpy(), ref2, mag2, TOL_F32, "call values")
    assert torch.equal(csa.plan_spmm(pl, Xd, ctx=ctx), Y)
    ctx.close()


def test_plan_probes_formats_and_modes(pl_graph):
    """Where the model proposes the format, a plan probes the plain pattern
    and several part counts; every mode yields a correct plan."""
    csr, rng = pl_graph
    F = 64
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, X, threads=THREADS)
    rp, ci = pattern_dev(csr)
    Xd = dev(X)
    ctx = csa.Context(0, None)
    with pytest.raises(csa.CsrError) as ei:
        csa.plan("spmm", rp, ci, None, Xd, mode="replay", ctx=ctx)
    assert "CSR_ERR_NO_CACHE_ENTRY" in str(ei.value)
    for mode in ("estimate", "probe", "auto", "replay"):
        pl = csa.plan("spmm", rp, ci, None, Xd, mode=mode, ctx=ctx)
        assert_close(csa.plan_spmm(pl, Xd, ctx=ctx).cpu().numpy(), ref, mag, TOL_F32, mode)
        print(f"mode {mode}: {pl}")
    ctx.close()


def test_plan_cache_file(tmp_path, pl_graph):
    csr, rng = pl_graph
    X = dev(rng.standard_normal((csr.n_cols, 32)).astype(np.float32))
    rp, ci = pattern_dev(csr)
    path = str(tmp_path / "plans.log")
    ctx = csa.Context(0, path)
    pl = csa.plan("spmm", rp, ci, None, X, ctx=ctx)
    Y = csa.plan_spmm(pl, X, ctx=ctx)
    ctx.close()
    text = open(path).read()
    assert "csrsa-plan v1" in text and f"{pl.signature:016x}" in text
    ctx2 = csa.Context(0, path)
    assert ctx2.cache_info()["entries"] >= 1
    pl2 = csa.plan("spmm", rp, ci, None, X, mode="replay", ctx=ctx2)
    assert pl2.choice() == pl.choice()
    assert torch.equal(csa.plan_spmm(pl2, X, ctx=ctx2), Y)
    ctx2.close()


@pytest.mark.parametrize("K", [4, 16, 64])
def test_plan_sddmm(pl_graph, K):
    csr, rng = pl_graph
    U = rng.standard_normal((csr.n_rows, K)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, K)).astype(np.float32)
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, threads=THREADS)
    rp, ci = pattern_dev(csr)
    Ud, Vd = dev(U), dev(V)
    ctx = csa.Context(0, None)
    pl = csa.plan("sddmm", rp, ci, Ud, Vd, ctx=ctx)
    out = csa.plan_sddmm(pl, Ud, Vd, ctx=ctx)
    e = assert_close(out.cpu().numpy(), ref, mag, TOL_F32, f"plan sddmm K={K}")
    print(f"plan sddmm K={K}: {pl} max err {e:.2e}")
    ctx.close()


def test_plan_skew_bf16():
    """bf16 features on the skew graph (30% empty rows and a row of 80,000
    entries): the plan's product against the oracle reading the same bf16
    values; an SDDMM plan on bf16 operands likewise."""
    csr = skew_graph(1)
    rng = np.random.default_rng(9)
    Xb = to_bf16_bits(rng.standard_normal((csr.n_cols, 64)).astype(np.float32))
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, oracle.bf16_to_f32(Xb), threads=THREADS)
    rp, ci = pattern_dev(csr)
    ctx = csa.Context(0, None)
    pl = csa.plan("spmm", rp, ci, dev(vals), bf16_dev(Xb), ctx=ctx)
    e = assert_close(csa.plan_spmm(pl, bf16_dev(Xb), ctx=ctx).cpu().numpy(), ref, mag, TOL_BF16, "bf16 plan")
    assert e <= TOL_F32
    print(f"skew bf16: {pl}")
    Ub = to_bf16_bits(rng.standard_normal((csr.n_rows, 32)).astype(np.float32))
    Vb = to_bf16_bits(rng.standard_normal((csr.n_cols, 32)).astype(np.float32))
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, oracle.bf16_to_f32(Ub), oracle.bf16_to_f32(Vb),
                            threads=THREADS)
    pl = csa.plan("sddmm", rp, ci, bf16_dev(Ub), bf16_dev(Vb), ctx=ctx)
    out = csa.plan_sddmm(pl, bf16_dev(Ub), bf16_dev(Vb), ctx=ctx)
    assert assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, "bf16 sddmm plan") <= TOL_F32
    ctx.close()


def test_plan_errors(pl_graph):
    csr, rng = pl_graph
    X = dev(rng.standard_normal((csr.n_cols, 64)).astype(np.float32))
    rp, ci = pattern_dev(csr)
    ctx = csa.Context(0, None)
    pl = csa.plan("spmm", rp, ci, None, X, ctx=ctx)
    lib = csa.load_library()
    # a plan of another op
    with pytest.raises(ValueError):
        csa.plan_sddmm(pl, X[:csr.n_rows], X, ctx=ctx)
    # X whose rows are not 16-byte aligned, under a plan that reads 4 values per lane
    if pl.parts == 1 and pl.schedule.vec == 4:
        Xs = torch.empty((csr.n_cols, 65), device="cuda")[:, 1:]
        Xs.copy_(X)
        with pytest.raises(csa.CsrError) as ei:
            csa.plan_spmm(pl, Xs, ctx=ctx)
        assert "CSR_ERR_SCHEDULE" in str(ei.value) or "CSR_ERR_ALIGN" in str(ei.value)
    # plan memory below csr_plan_size's figure
    p, _ = csa.make_problem("spmm", rp, ci, None, X)
    ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    p.stream = torch.cuda.current_stream().cuda_stream
    need, need_ws = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.csr_plan_size(ctx.handle, ctypes.byref(p), ctypes.byref(need), ctypes.byref(need_ws)) == 0
    assert need.value > 256
    mem = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    desc = csa.CsrPlan()
    rc = lib.csr_plan_create(ctx.handle, ctypes.byref(p), 0, mem.data_ptr(), need.value - 256, ctypes.byref(desc))
    assert rc == -5  # CSR_ERR_WORKSPACE
    torch.cuda.synchronize()
    ctx.close()


# ---------------------------------------------------------------------------
# degree classes (short rows packed slot-major by class, the other rows as a
# CSR of their own), forced through the plan log: every schedule of the
# long rows' product, both short thresholds
# ---------------------------------------------------------------------------

def _long_rows(csr, E):
    """The long rows' CSR of the degree classes (rows of E or more entries;
    the packed and the empty rows have none), from the pattern."""
    deg = np.diff(csr.row_ptr)
    keep = deg >= E
    rp = np.zeros(csr.n_rows + 1, np.int32)
    rp[1:] = np.cumsum(np.where(keep, deg, 0))
    ci = np.concatenate([csr.col_idx[csr.row_ptr[r]:csr.row_ptr[r + 1]] for r in np.nonzero(keep)[0]]
                        + [np.zeros(0, np.int32)]).astype(np.int32)
    return rp, ci


def _forced_plan(tmp_path, name, sig, E, s, rp, ci, operands):
    path = str(tmp_path / f"{name}.log")
    with open(path, "w") as f:
        f.write(f"csrsa-plan v1 {sig:016x} parts=0 whole={E} op={s.op} map={s.mapping} vec={s.vec} "
                f"w={s.group_lanes} nv={s.passes} chunk={s.chunk_items} long={s.long_row} flags={s.flags} "
                f"us=1.000\n")
    ctx = csa.Context(0, path)
    pl = csa.plan("spmm", rp, ci, *operands, mode="replay", ctx=ctx)
    return pl, ctx


def _mixed_graph(seed):
    """2,000 rows: a quarter empty, many single entries, short rows of 2 to 31
    entries, a few long rows and one of 6,000 (split over merge-path chunks)."""
    rng = np.random.default_rng(seed)
    n, n_cols = 2000, 20_000
    kind = rng.random(n)
    deg = np.where(kind < 0.25, 0, np.where(kind < 0.55, 1, rng.integers(2, 32, n)))
    deg[rng.choice(n, 20, replace=False)] = rng.integers(40, 600, 20)
    deg[rng.integers(0, n)] = 6000
    return graphs.csr_from_degrees(deg, n_cols, rng)


@pytest.mark.parametrize("E", [8, 32])
@pytest.mark.parametrize("F", [4, 24, 130])
def test_classes_every_long_schedule(tmp_path, E, F):
    csr = _mixed_graph(11)
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    rp, ci = pattern_dev(csr)
    vd, Xd = dev(vals), dev(X)
    ctx0 = csa.Context(0, None)
    sig = csa.plan("spmm", rp, ci, vd, Xd, ctx=ctx0).signature
    ctx0.close()
    lrp, lci = _long_rows(csr, E)
    lrp_d, lci_d = dev(lrp), dev(lci)
    q, _ = csa.make_problem("spmm", lrp_d, lci_d, dev(np.ones(len(lci), np.float32)), Xd)
    c, sm, mx = csa.degree_histogram(lrp_d)
    scheds = csa.candidates(q, c + sm + [mx])
    assert len(scheds) >= 3
    v2 = rng.standard_normal(csr.nnz).astype(np.float32)
    ref2, mag2 = oracle.spmm(csr.row_ptr, csr.col_idx, v2, X, threads=THREADS)
    for k, s in enumerate(scheds):
        pl, ctx = _forced_plan(tmp_path, f"s{k}", sig, E, s, rp, ci, (vd, Xd))
        assert pl.layout == "classes" and pl.whole_below == E and bytes(pl.schedule) == bytes(s)
        b = pl.desc.bkt
        deg = np.diff(csr.row_ptr)
        assert b.n_short == int(((deg >= 1) & (deg < E)).sum()) and b.nnz_long == len(lci)
        Y = csa.plan_spmm(pl, Xd, ctx=ctx)
        what = f"E={E} F={F} {s}"
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, what)
        # the same plan again: bit for bit; this call's own values
        assert torch.equal(csa.plan_spmm(pl, Xd, ctx=ctx), Y)
        assert_close(csa.plan_spmm(pl, Xd, vals=dev(v2), ctx=ctx).cpu().numpy(), ref2, mag2, TOL_F32, what)
        ctx.close()


def test_classes_unit_values_bf16_and_infinities(tmp_path):
    """Ones for values, bf16 features, and an infinite feature that only
    padding slots would meet: it must not turn into NaN (padding is skipped,
    not multiplied by 0)."""
    csr = _mixed_graph(13)
    rng = np.random.default_rng(14)
    rp, ci = pattern_dev(csr)
    F = 64
    Xb = to_bf16_bits(rng.standard_normal((csr.n_cols, F)).astype(np.float32))
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, oracle.bf16_to_f32(Xb), threads=THREADS)
    ctx0 = csa.Context(0, None)
    sig = csa.plan("spmm", rp, ci, None, bf16_dev(Xb), ctx=ctx0).signature
    ctx0.close()
    s = csa.default_schedule(csa.make_problem("spmm", rp, ci, None, bf16_dev(Xb))[0])
    pl, ctx = _forced_plan(tmp_path, "bf16", sig, 8, s, rp, ci, (None, bf16_dev(Xb)))
    assert pl.layout == "classes"
    e = assert_close(csa.plan_spmm(pl, bf16_dev(Xb), ctx=ctx).cpu().numpy(), ref, mag, TOL_BF16, "bf16 classes")
    assert e <= TOL_F32
    ctx.close()
    # an infinite feature in a row that no stored entry points at
    used = np.zeros(csr.n_cols, bool)
    used[csr.col_idx] = True
    unused = int(np.nonzero(~used)[0][0])
    X = rng.standard_normal((csr.n_cols, 8)).astype(np.float32)
    X[unused] = np.inf
    ctx0 = csa.Context(0, None)
    sig = csa.plan("spmm", rp, ci, None, dev(X), ctx=ctx0).signature
    ctx0.close()
    s = csa.default_schedule(csa.make_problem("spmm", rp, ci, None, dev(X))[0])
    pl, ctx = _forced_plan(tmp_path, "inf", sig, 32, s, rp, ci, (None, dev(X)))
    Y = csa.plan_spmm(pl, dev(X), ctx=ctx).cpu().numpy()
    assert np.isfinite(Y).all()
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, X, threads=THREADS)
    assert_close(Y, ref, mag, TOL_F32, "unit values")
    ctx.close()
    # the plan's own choice on a graph whose short rows hold most entries
    # (the degree classes are among the layouts it probes)
    ctx = csa.Context(0, None)
    Xf = rng.standard_normal((csr.n_cols, 8)).astype(np.float32)
    pl = csa.plan("spmm", rp, ci, None, dev(Xf), ctx=ctx)
    print(f"mixed graph F=8: {pl}")
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, Xf, threads=THREADS)
    assert_close(csa.plan_spmm(pl, dev(Xf), ctx=ctx).cpu().numpy(), ref, mag, TOL_F32, "auto")
    ctx.close()


def test_classes_on_the_skew_stress_graph():
    """The 1M-row Zipf graph (675k single-entry rows): the plan weighs the
    degree classes among its layouts; whichever it picks matches the oracle,
    and the classes at both thresholds do too."""
    from synth import configs

    csr = configs.config_pattern("c4")
    rp, ci = pattern_dev(csr)
    vals = configs.config_dense("c4", "vals", csr)
    X = configs.config_dense("c4", "X", csr, 4)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    vd, Xd = dev(vals), dev(X)
    ctx = csa.Context(0, None)
    pl = csa.plan("spmm", rp, ci, vd, Xd, ctx=ctx)
    print(f"c4 F=4 plan: {pl}")
    assert_close(csa.plan_spmm(pl, Xd, ctx=ctx).cpu().numpy(), ref, mag, TOL_F32, "auto plan")
    ctx.close()


def test_plan_build_every_layout(pl_graph):
    """csr_plan_build: the plain pattern, the format at several part counts
    and thresholds, and the degree classes at both thresholds, each with the
    selector's schedule for its product, all against the oracle; an explicit
    schedule is taken as given; layouts outside the rules are refused."""
    csr, rng = pl_graph
    F = 64
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    rp, ci = pattern_dev(csr)
    vd, Xd = dev(vals), dev(X)
    ctx = csa.Context(0, None)
    for layout in ((1, 0), (4, 0), (16, 64), (64, 0), (0, 8), (0, 32)):
        pl = csa.plan("spmm", rp, ci, vd, Xd, layout=layout, ctx=ctx)
        assert (pl.parts, pl.whole_below) == layout
        assert_close(csa.plan_spmm(pl, Xd, ctx=ctx).cpu().numpy(), ref, mag, TOL_F32, f"layout {layout}")
        print(f"layout {layout}: {pl}")
    # an explicit schedule for the plain pattern
    s = csa.candidates(csa.make_problem("spmm", rp, ci, vd, Xd)[0])[1]
    pl = csa.plan("spmm", rp, ci, vd, Xd, layout=(1, 0), schedule=s, ctx=ctx)
    assert bytes(pl.schedule) == bytes(s)
    assert_close(csa.plan_spmm(pl, Xd, ctx=ctx).cpu().numpy(), ref, mag, TOL_F32, "given schedule")
    for bad in ((3, 0), (512, 0), (0, 6), (0, 128), (-1, 0), (8, -1)):
        with pytest.raises(csa.CsrError) as ei:
            csa.plan("spmm", rp, ci, vd, Xd, layout=bad, ctx=ctx)
        assert "CSR_ERR_SHAPE" in str(ei.value), bad
    U = dev(rng.standard_normal((csr.n_rows, 16)).astype(np.float32))
    V = dev(rng.standard_normal((csr.n_cols, 16)).astype(np.float32))
    with pytest.raises(csa.CsrError) as ei:
        csa.plan("sddmm", rp, ci, U, V, layout=(0, 8), ctx=ctx)  # degree classes serve SpMM
    assert "CSR_ERR_SHAPE" in str(ei.value)
    sd = csa.default_schedule(csa.make_problem("sddmm", rp, ci, U, V)[0])
    with pytest.raises(csa.CsrError) as ei:
        csa.plan("spmm", rp, ci, vd, Xd, layout=(1, 0), schedule=sd, ctx=ctx)  # a schedule of another op
    assert "CSR_ERR_SCHEDULE" in str(ei.value)
    ctx.close()
