"""GPU parity: every mapping and lane layout of every op against the CPU
oracle on seeded graphs that span many chunks, with skew, empty rows, a row
long enough to be split over more than 64 merge-path chunks, ragged widths and
strided operands; plus the bit-exact cases (identity pattern, empty rows,
pass-through of row_ptr / col_idx, replay determinism, integer bookkeeping)."""

import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
import oracle  # noqa: E402
from synth import graphs, to_bf16_bits  # noqa: E402
from synth.graphs import CSR  # noqa: E402
from gpu_util import TOL_BF16, TOL_F32, assert_close, bf16_dev, dev  # noqa: E402

_ffi = csa._ffi


def skew_graph(seed, n_rows=3000, n_cols=100_000, giant=80_000):
    """30% empty rows, short Poisson rows, medium rows, a few long rows and one
    giant row (split over > 64 chunks of 1024 items)."""
    rng = np.random.default_rng(seed)
    kind = rng.random(n_rows)
    deg = np.where(kind < 0.3, 0, rng.poisson(3, n_rows))
    mid = (kind > 0.8) & (kind < 0.95)
    deg[mid] = rng.integers(50, 300, mid.sum())
    longr = rng.choice(n_rows, 5, replace=False)
    deg[longr] = rng.integers(2000, 5000, 5)
    deg[rng.integers(0, n_rows)] = giant
    deg = np.minimum(deg, n_cols)
    return graphs.csr_from_degrees(deg, n_cols, rng)


def dup_graph(seed):
    """Unsorted columns with duplicate entries."""
    rng = np.random.default_rng(seed)
    return graphs.random_small_graph(700, 900, 0.02, rng, empty_frac=0.2, allow_dup=True)


def pattern_dev(csr):
    return dev(csr.row_ptr), dev(csr.col_idx)


def schedules(problem, thorough=True):
    """The default schedule and its variants: both mappings, every chunk size,
    whole-wave / per-group / default long-row thresholds, halved group width."""
    base = csa.default_schedule(problem)
    layouts = [(base.group_lanes, base.passes)]
    W2, nv2 = base.group_lanes // 2, base.passes * 2
    # the halved layout when its pass count is the fewest supported that covers the width
    need = -(-problem.width // max(1, W2 * base.vec))
    if W2 >= 1 and nv2 in (2, 4, 6, 8, 12, 16) and min(v for v in (1, 2, 3, 4, 5, 6, 8, 12, 16, 99) if v >= need) == nv2:
        layouts.append((W2, nv2))
    out = []
    for W, nv in layouts:
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.group_lanes, s.passes = W, nv
        s.mapping, s.chunk_items, s.long_row = csa.MAP_ROWGROUP, 0, 0
        out.append(s)
        chunks = (256, 512, 1024) if thorough else (512,)
        G = 64 // W
        lrs = sorted({0, G * 4, 1 << 30}) if thorough else [G * 4]
        for D in chunks:
            for lr in lrs:
                s = csa.CsrSchedule.from_buffer_copy(bytes(base))
                s.group_lanes, s.passes = W, nv
                s.mapping, s.chunk_items, s.long_row = csa.MAP_MERGEPATH, D, lr
                out.append(s)
    # SpMM row groups with wide lanes (4 floats per lane at any 4-byte alignment)
    if problem.op == _ffi.OP_SPMM and problem.width >= 4 and problem.dtype == _ffi.DTYPE_F32:
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.mapping, s.vec, s.group_lanes, s.chunk_items, s.long_row = csa.MAP_ROWGROUP, 4, 64, 0, 0
        need = -(-problem.width // 256)
        s.passes = min(v for v in (1, 2, 3, 4, 5, 6, 8, 12, 16) if v >= need)
        s.flags = csa.SCHED_WIDE
        out.append(s)
    # entry-parallel segmented scan for small widths (SpMM, SDDMM)
    if problem.op in (_ffi.OP_SPMM, _ffi.OP_SDDMM) and problem.width <= 4 * base.vec:
        for D in ((256, 512, 1024) if thorough else (512,)):
            s = csa.CsrSchedule.from_buffer_copy(bytes(base))
            s.mapping, s.group_lanes, s.chunk_items, s.long_row = csa.MAP_SEGSCAN, 1, D, 0
            s.passes = -(-problem.width // base.vec)
            out.append(s)
    return out


def sched_id(s):
    return f"m{s.mapping}-w{s.group_lanes}-nv{s.passes}-v{s.vec}-d{s.chunk_items}-lr{s.long_row}-f{s.flags}"


# ---------------------------------------------------------------------------
# SpMM
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def skew():
    return skew_graph(1)


@pytest.mark.parametrize("F", [1, 4, 32, 64, 602])
def test_spmm_every_schedule(skew, F):
    csr = skew
    rng = np.random.default_rng(F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    v, Xd = dev(vals), dev(X)
    p, out = csa.make_problem("spmm", rp, ci, v, Xd)
    for s in schedules(p):
        Y = csa.spmm(rp, ci, v, Xd, schedule=s)
        torch.cuda.synchronize()
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))
    Y = csa.spmm(rp, ci, v, Xd)  # automatic selection
    assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, "auto")


# 601 and 777 floats one at a time: 12 and 16 passes of 64 lanes, the last 2 and 3 all masked
@pytest.mark.parametrize("F", [2, 3, 5, 7, 8, 16, 17, 100, 128, 256, 300, 601, 777, 1024])
def test_spmm_widths(F):
    csr = skew_graph(2, n_rows=1500, n_cols=20_000, giant=9000)
    rng = np.random.default_rng(100 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("spmm", rp, ci, dev(vals), dev(X))
    for s in schedules(p, thorough=False):
        Y = csa.spmm(rp, ci, dev(vals), dev(X), schedule=s)
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))


def test_spmm_strided_and_unit_values():
    csr = skew_graph(3, n_rows=800, n_cols=5000, giant=3000)
    rng = np.random.default_rng(3)
    F, ldx, ldy = 24, 40, 36
    Xbig = rng.standard_normal((csr.n_cols, ldx)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, Xbig[:, :F])
    rp, ci = pattern_dev(csr)
    Xd = dev(Xbig)[:, :F]
    Ybig = torch.full((csr.n_rows, ldy), 7.0, device="cuda")
    Y = Ybig[:, :F]
    p, _ = csa.make_problem("spmm", rp, ci, None, Xd, out=Y)
    for s in schedules(p, thorough=False):
        csa.spmm(rp, ci, None, Xd, out=Y, schedule=s)
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))
        assert torch.all(Ybig[:, F:] == 7.0), "columns beyond F must not be written"


def test_spmm_duplicates_unsorted():
    csr = dup_graph(4)
    rng = np.random.default_rng(4)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, 33)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("spmm", rp, ci, dev(vals), dev(X))
    for s in schedules(p, thorough=False):
        Y = csa.spmm(rp, ci, dev(vals), dev(X), schedule=s)
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))


# ---------------------------------------------------------------------------
# attention (scores given)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("F", [1, 4, 32, 64, 100, 601])
def test_attention_every_schedule(skew, F):
    csr = skew
    rng = np.random.default_rng(200 + F)
    sc = (2 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.uniform(-1, 1, (csr.n_cols, F)).astype(np.float32)
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, 1.0, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    s_d, V_d = dev(sc), dev(V)
    p, _ = csa.make_problem("attention", rp, ci, s_d, V_d)
    for s in schedules(p):
        out = csa.attention(rp, ci, s_d, V_d, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))
    out = csa.attention(rp, ci, s_d, V_d)
    assert_close(out.cpu().numpy(), ref, mag, TOL_F32, "auto")


@pytest.mark.parametrize("scale", [0.125, 3.0])
def test_attention_scale_and_duplicates(scale):
    csr = dup_graph(5)
    rng = np.random.default_rng(5)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, 16)).astype(np.float32)
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, scale)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("attention", rp, ci, dev(sc), dev(V), scale=scale)
    for s in schedules(p, thorough=False):
        out = csa.attention(rp, ci, dev(sc), dev(V), scale=scale, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))


def test_attention_shift_invariance_large_offsets(skew):
    """+-1000 added per row (exact in fp32 for scores on a 2^-10 grid): the
    max subtraction keeps exp finite and the result matches the oracle."""
    csr = skew
    rng = np.random.default_rng(6)
    base = (np.round(rng.standard_normal(csr.nnz) * 1024) / 1024).astype(np.float32)
    shift = np.repeat(rng.choice([-1000.0, 0.0, 1000.0], csr.n_rows), csr.degrees()).astype(np.float32)
    sc = base + shift
    V = rng.standard_normal((csr.n_cols, 8)).astype(np.float32)
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, base, V)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("attention", rp, ci, dev(sc), dev(V))
    for s in schedules(p, thorough=False):
        out = csa.attention(rp, ci, dev(sc), dev(V), schedule=s)
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o))
        assert_close(o, ref, mag, TOL_F32, sched_id(s))


def test_c1_attention_workload():
    from synth import configs

    c = configs.make_config("c1")
    csr = c["csr"]
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, c["scores"], c["V"])
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("attention", rp, ci, dev(c["scores"]), dev(c["V"]))
    for s in schedules(p):
        out = csa.attention(rp, ci, dev(c["scores"]), dev(c["V"]), schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))


def test_p4_size_attention():
    from synth import configs

    c = configs.make_config("p4")
    csr = c["csr"]
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, c["scores"], c["V"])
    rp, ci = pattern_dev(csr)
    out = csa.attention(rp, ci, dev(c["scores"]), dev(c["V"]))
    assert_close(out.cpu().numpy(), ref, mag, TOL_F32)


# ---------------------------------------------------------------------------
# SDDMM
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K", [1, 4, 32, 64, 128, 601, 602])
def test_sddmm_every_schedule(K):
    csr = skew_graph(7, n_rows=2000, n_cols=30_000, giant=25_000)
    rng = np.random.default_rng(300 + K)
    U = rng.standard_normal((csr.n_rows, K)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, K)).astype(np.float32)
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    Ud, Vd = dev(U), dev(V)
    p, _ = csa.make_problem("sddmm", rp, ci, Ud, Vd)
    for s in schedules(p):
        out = csa.sddmm(rp, ci, Ud, Vd, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))
    out = csa.sddmm(rp, ci, Ud, Vd)
    assert_close(out.cpu().numpy(), ref, mag, TOL_F32, "auto")


# ---------------------------------------------------------------------------
# multi-head attention (bf16 in, fp32 accumulate)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,D", [(8, 64), (2, 8), (1, 512), (4, 32), (3, 16)])
def test_mha_schedules(H, D):
    csr = skew_graph(8, n_rows=1200, n_cols=30_000, giant=20_000)
    rng = np.random.default_rng(400 + H * D)
    Q = to_bf16_bits(rng.standard_normal((csr.n_rows, H, D)).astype(np.float32))
    K = to_bf16_bits(rng.standard_normal((csr.n_cols, H, D)).astype(np.float32))
    V = to_bf16_bits(rng.standard_normal((csr.n_cols, H, D)).astype(np.float32))
    scale = 1.0 / np.sqrt(D)
    ref, mag, _ = oracle.mha(csr.row_ptr, csr.col_idx, Q, K, V, scale, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    p, _ = csa.make_problem("mha", rp, ci, Qd, Kd, Vd, scale=scale)
    base = csa.default_schedule(p)
    scheds = []
    for mapping, D_items in ((csa.MAP_ROWGROUP, 0), (csa.MAP_MERGEPATH, 256), (csa.MAP_MERGEPATH, 512),
                             (csa.MAP_MERGEPATH, 1024)):
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.mapping, s.chunk_items = mapping, D_items
        scheds.append(s)
    for s in scheds:
        out = csa.mha_attention(rp, ci, Qd, Kd, Vd, scale=scale, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, sched_id(s))
        # fp32 accumulation keeps the error far below the bf16 tolerance
        assert_close(out.cpu().numpy(), ref, mag, 1e-4, sched_id(s))
    out = csa.mha_attention(rp, ci, Qd, Kd, Vd, scale=scale)
    assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, "auto")


# ---------------------------------------------------------------------------
# exact cases
# ---------------------------------------------------------------------------

def test_identity_pattern_bit_exact():
    n, F = 5000, 64
    rng = np.random.default_rng(9)
    rp = np.arange(n + 1, dtype=np.int32)
    ci = np.arange(n, dtype=np.int32)
    V = rng.standard_normal((n, F)).astype(np.float32)
    sc = (30 * rng.standard_normal(n)).astype(np.float32)
    rpd, cid, Vd = dev(rp), dev(ci), dev(V)
    p, _ = csa.make_problem("attention", rpd, cid, dev(sc), Vd)
    for s in schedules(p):
        out = csa.attention(rpd, cid, dev(sc), Vd, schedule=s).cpu().numpy()
        assert np.array_equal(out.view(np.uint32), V.view(np.uint32)), sched_id(s)
        Y = csa.spmm(rpd, cid, None, Vd, schedule=_as_op(s, 1)).cpu().numpy()
        assert np.array_equal(Y.view(np.uint32), V.view(np.uint32)), sched_id(s)
    Q = to_bf16_bits(rng.standard_normal((n, 8, 64)).astype(np.float32))
    Vb = to_bf16_bits(rng.standard_normal((n, 8, 64)).astype(np.float32))
    out = csa.mha_attention(rpd, cid, bf16_dev(Q), bf16_dev(Q), bf16_dev(Vb)).cpu().numpy()
    want = (Vb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(out, want)


def _as_op(s, op):
    t = csa.CsrSchedule.from_buffer_copy(bytes(s))
    t.op = op
    return t


def test_empty_rows_positive_zero_and_empty_graph():
    n = 4000
    rng = np.random.default_rng(10)
    deg = np.where(rng.random(n) < 0.5, 0, rng.integers(1, 9, n))
    csr = graphs.csr_from_degrees(deg, 3000, rng)
    V = rng.standard_normal((3000, 20)).astype(np.float32)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("attention", rp, ci, dev(sc), dev(V))
    empty = csr.degrees() == 0
    for s in schedules(p, thorough=False):
        out = torch.full((n, 20), float("nan"), device="cuda")
        csa.attention(rp, ci, dev(sc), dev(V), out=out, schedule=s)
        o = out.cpu().numpy()
        assert np.all(o[empty].view(np.uint32) == 0), sched_id(s)
        Y = torch.full((n, 20), float("nan"), device="cuda")
        csa.spmm(rp, ci, dev(sc), dev(V), out=Y, schedule=_as_op(s, 1))
        assert np.all(Y.cpu().numpy()[empty].view(np.uint32) == 0)
    # no entries at all
    rp0 = dev(np.zeros(n + 1, np.int32))
    ci0 = torch.empty(0, dtype=torch.int32, device="cuda")
    for fn, args in ((csa.spmm, (None, dev(V))), (csa.attention, (torch.empty(0, device="cuda"), dev(V)))):
        out = torch.full((n, 20), float("nan"), device="cuda")
        fn(rp0, ci0, *args, out=out)
        assert torch.all(out == 0) and not torch.any(torch.signbit(out))
    out = csa.sddmm(rp0, ci0, dev(rng.standard_normal((n, 20)).astype(np.float32)), dev(V))
    assert out.numel() == 0
    # no rows at all
    Y = csa.spmm(dev(np.zeros(1, np.int32)), ci0, None, dev(V))
    assert Y.shape == (0, 20)


def test_inputs_pass_through_and_replay_determinism(skew):
    csr = skew
    rng = np.random.default_rng(11)
    sc = rng.standard_normal(csr.nnz).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, 32)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    sd, Vd = dev(sc), dev(V)
    p, _ = csa.make_problem("attention", rp, ci, sd, Vd)
    for s in schedules(p, thorough=False):
        a = csa.attention(rp, ci, sd, Vd, schedule=s).cpu().numpy()
        b = csa.attention(rp, ci, sd, Vd, schedule=s).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), sched_id(s)
    assert np.array_equal(rp.cpu().numpy(), csr.row_ptr)
    assert np.array_equal(ci.cpu().numpy(), csr.col_idx)
    assert np.array_equal(sd.cpu().numpy(), sc) and np.array_equal(Vd.cpu().numpy(), V)


# ---------------------------------------------------------------------------
# integer bookkeeping, selector and cache
# ---------------------------------------------------------------------------

def test_degree_histogram_and_partition_bit_exact(skew):
    csr = skew
    rp = dev(csr.row_ptr)
    counts, sums, mx = csa.degree_histogram(rp)
    oc, osum, omx = oracle.degree_histogram(csr.row_ptr)
    assert counts == oc.tolist() and sums == osum.tolist() and mx == omx
    for D in (1, 7, 256, 1024, 5000):
        coords = csa.merge_path_partition(rp, csr.nnz, D).cpu().numpy()
        x, y = oracle.merge_path_partition(csr.row_ptr, D)
        assert np.array_equal(coords[:, 0], x) and np.array_equal(coords[:, 1], y)


def test_select_replay_and_cache_file(tmp_path, skew):
    csr = skew
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, 64)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    vd, Xd = dev(vals), dev(X)
    path = str(tmp_path / "cache.log")
    ctx = csa.Context(0, path)
    s1, sig1 = csa.select("spmm", rp, ci, vd, Xd, ctx=ctx)
    s2, sig2 = csa.select("spmm", rp, ci, vd, Xd, ctx=ctx)  # cache hit
    s3, sig3 = csa.select("spmm", rp, ci, vd, Xd, mode="replay", ctx=ctx)
    assert sig1 == sig2 == sig3 and bytes(s1) == bytes(s2) == bytes(s3)
    assert ctx.cache_info()["entries"] == 1
    ctx.close()
    ctx2 = csa.Context(0, path)  # reload from the log
    s4, sig4 = csa.select("spmm", rp, ci, vd, Xd, mode="replay", ctx=ctx2)
    assert sig4 == sig1 and bytes(s4) == bytes(s1)
    Y = csa.spmm(rp, ci, vd, Xd, schedule=s4, ctx=ctx2)
    assert_close(Y.cpu().numpy(), ref, mag, TOL_F32)
    # a different width is a different signature: replay-only misses
    X2 = dev(rng.standard_normal((csr.n_cols, 48)).astype(np.float32))
    with pytest.raises(csa.CsrError) as ei:
        csa.select("spmm", rp, ci, vd, X2, mode="replay", ctx=ctx2)
    assert ei.value.code == _ffi.CSR_ERR_NO_CACHE_ENTRY
    ctx2.close()


def test_probe_failure_falls_back_to_default(monkeypatch, skew):
    csr = skew
    rp, ci = pattern_dev(csr)
    X = dev(np.ones((csr.n_cols, 16), np.float32))
    monkeypatch.setenv("CSRSA_FAIL_PROBE", "1")
    ctx = csa.Context(0, None)
    s, _ = csa.select("spmm", rp, ci, None, X, ctx=ctx)
    p, _ = csa.make_problem("spmm", rp, ci, None, X)
    assert bytes(s) == bytes(csa.default_schedule(p))
    assert ctx.cache_info()["entries"] == 0  # a fallback is not cached
    ctx.close()


def test_error_codes(skew):
    csr = skew
    lib = csa.load_library()
    ctx = csa.default_context(0)
    rp, ci = pattern_dev(csr)
    X = dev(np.ones((csr.n_cols, 16), np.float32))
    Y = torch.empty((csr.n_rows, 16), device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    n, m, nnz = csr.n_rows, csr.n_cols, csr.nnz

    def call(**kw):
        a = dict(rp=rp.data_ptr(), ci=ci.data_ptr(), X=X.data_ptr(), F=16, ldx=16, Y=Y.data_ptr(), ldy=16,
                 ws=ws.data_ptr(), wsb=ws.numel(), n=n, m=m, nnz=nnz, sched=None, dt=0)
        a.update(kw)
        return lib.csr_spmm(ctx.handle, a["n"], a["m"], a["nnz"], a["rp"], a["ci"], None, a["X"], a["dt"], a["F"],
                            a["ldx"], a["Y"], a["ldy"], a["sched"], a["ws"], a["wsb"], st)

    assert call() == 0
    assert call(rp=None) == -1
    assert call(X=None) == -1
    assert call(F=0) == -2
    assert call(ldx=8) == -2
    assert call(n=-1) == -2
    assert call(X=X.data_ptr() + 2) == -4
    assert call(wsb=16) == -5
    assert call(ws=ws.data_ptr() + 64) == -4
    assert call(dt=7) == -3                                   # unknown dtype
    assert call(dt=1, F=15, ldx=16) == -2                     # bf16 with an odd width
    assert call(dt=1, F=16, ldx=15) == -4                     # bf16 with an odd leading dimension
    assert call(dt=1, X=X.data_ptr() + 2) == -4               # bf16 rows not 4-byte aligned
    p, _ = csa.make_problem("spmm", rp, ci, None, X, out=Y)
    s = csa.default_schedule(p)
    s.op = _ffi.OP_ATTENTION
    assert call(sched=ctypes.byref(s)) == -7
    s = csa.default_schedule(p)
    s.chunk_items = 300
    assert call(sched=ctypes.byref(s)) == -7
    s = csa.default_schedule(p)
    s.vec = 4
    assert call(F=6, ldx=6, ldy=6, sched=ctypes.byref(s)) == -7
    torch.cuda.synchronize()


def test_validation_flag_rejects_bad_columns():
    rng = np.random.default_rng(13)
    csr = graphs.random_small_graph(200, 300, 0.05, rng)
    bad = csr.col_idx.copy()
    bad[len(bad) // 2] = 300  # out of range
    rp, ci = dev(csr.row_ptr), dev(bad)
    X = dev(np.ones((300, 8), np.float32))
    ctx = csa.Context(0, None, flags=csa.CTX_VALIDATE)
    with pytest.raises(csa.CsrError) as ei:
        csa.spmm(rp, ci, None, X, ctx=ctx)
    assert ei.value.code == -6
    Y = csa.spmm(rp, dev(csr.col_idx), None, X, ctx=ctx)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, np.ones((300, 8), np.float32))
    assert_close(Y.cpu().numpy(), ref, mag)
    ctx.close()


@pytest.mark.parametrize("corrupt", ["start", "end", "order"])
def test_validation_flag_rejects_bad_row_ptr(corrupt):
    """A validating context rejects a row_ptr that breaks the CSR invariants
    (row_ptr[0] = 0, row_ptr[n_rows] = nnz, non-decreasing) before any
    product kernel runs, for SpMM, SDDMM, attention and the row softmax; the
    same context then runs the intact pattern."""
    rng = np.random.default_rng(17)
    csr = graphs.random_small_graph(200, 300, 0.05, rng)
    bad = csr.row_ptr.copy()
    if corrupt == "start":
        bad[0] = 1
    elif corrupt == "end":
        bad[-1] = csr.nnz - 1
    else:
        i = int(np.argmax(np.diff(bad) > 0)) + 1  # a row boundary inside the array with a non-empty row before it
        bad[i] = bad[i - 1] - 1 if bad[i - 1] > 0 else bad[i + 1] + 1
        assert (np.diff(bad) < 0).any()
    assert 0 <= bad.min() and bad.max() <= csr.nnz  # every value stays inside the entry arrays
    rp_bad, rp, ci = dev(bad), dev(csr.row_ptr), dev(csr.col_idx)
    X = dev(rng.standard_normal((300, 8)).astype(np.float32))
    U = dev(rng.standard_normal((200, 8)).astype(np.float32))
    sc = dev(rng.standard_normal(csr.nnz).astype(np.float32))
    ctx = csa.Context(0, None, flags=csa.CTX_VALIDATE)
    try:
        for call in (lambda r: csa.spmm(r, ci, None, X, ctx=ctx),
                     lambda r: csa.sddmm(r, ci, U, X, ctx=ctx),
                     lambda r: csa.attention(r, ci, sc, X, ctx=ctx),
                     lambda r: csa.row_softmax(r, sc, ctx=ctx)):
            with pytest.raises(csa.CsrError) as ei:
                call(rp_bad)
            assert ei.value.code == -6, corrupt
            call(rp)  # the intact pattern passes the same checks
        Y = csa.spmm(rp, ci, None, X, ctx=ctx)
        ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, None, X.cpu().numpy())
        assert_close(Y.cpu().numpy(), ref, mag)
    finally:
        ctx.close()


# ---------------------------------------------------------------------------
# unfused pipeline: row softmax and SDDMM -> row-softmax -> SpMM
# ---------------------------------------------------------------------------

def short_rows_graph(seed):
    """Mostly empty and one-entry rows with a few long ones: hundreds of rows
    per merge-path chunk, runs of empty rows inside a lane's entries."""
    rng = np.random.default_rng(seed)
    n = 20_000
    deg = np.where(rng.random(n) < 0.4, 0, 1 + rng.poisson(0.3, n))
    deg[rng.choice(n, 4, replace=False)] = rng.integers(700, 3000, 4)
    return graphs.csr_from_degrees(deg, 50_000, rng)


def chunk_edge_graph(seed):
    """Rows of 255, 256, 257, 511, 512, 513 and 1024 entries (either side of
    the chunk sizes, where a row stops being kept whole by one chunk) between
    runs of short and empty rows."""
    rng = np.random.default_rng(seed)
    deg = []
    for L in (255, 256, 257, 511, 512, 513, 1024) * 6:
        deg += [L] + list(rng.integers(0, 6, rng.integers(0, 40)))
    return graphs.csr_from_degrees(np.array(deg), 5000, rng)


@pytest.mark.parametrize("graph", ["skew", "short", "edges"])
@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_row_softmax_every_schedule(skew, graph, scale):
    csr = {"skew": lambda: skew, "short": lambda: short_rows_graph(501), "edges": lambda: chunk_edge_graph(502)}[graph]()
    rng = np.random.default_rng(500)
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    _, _, ref = oracle.attention(csr.row_ptr, csr.col_idx, sc, np.zeros((csr.n_cols, 1), np.float32), scale,
                                 want_probs=True, threads=oracle.default_threads())
    rp = dev(csr.row_ptr)
    sd = dev(sc)
    p, _ = csa.make_problem("row_softmax", rp, None, sd, scale=scale)
    base = csa.default_schedule(p)
    scheds = csa.candidates(p)
    for D in (256, 512):
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.mapping, s.group_lanes, s.long_row, s.chunk_items = csa.MAP_MERGEPATH, 1, 32, D
        scheds.append(s)
    for D in (256, 512):
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.mapping, s.group_lanes, s.long_row, s.chunk_items = csa.MAP_SEGSCAN, 1, 0, D
        scheds.append(s)
    assert {s.mapping for s in scheds} == {csa.MAP_MERGEPATH, csa.MAP_SEGSCAN}
    for s in scheds:
        out = csa.row_softmax(rp, sd, scale=scale, schedule=s).cpu().numpy()
        err = np.max(np.abs(out.astype(np.float64) - ref) / ref)
        assert err < 1e-5, (sched_id(s), err)
        sums = np.add.reduceat(out.astype(np.float64), csr.row_ptr[:-1][csr.degrees() > 0])
        assert np.max(np.abs(sums - 1)) < 1e-5
    # in place
    x = dev(sc)
    csa.row_softmax(rp, x, scale=scale, out=x)
    assert np.max(np.abs(x.cpu().numpy() - ref) / ref) < 1e-5


def test_attention_pipeline_unfused_equals_fused():
    csr = skew_graph(14, n_rows=2000, n_cols=20_000, giant=12_000)
    rng = np.random.default_rng(14)
    d, F = 32, 48
    Q = rng.standard_normal((csr.n_rows, d)).astype(np.float32)
    K = rng.standard_normal((csr.n_cols, d)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    scale = 1.0 / np.sqrt(d)
    # oracle: SDDMM then softmax attention over those scores, in float64
    scores, _ = oracle.sddmm(csr.row_ptr, csr.col_idx, Q, K, threads=oracle.default_threads())
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, scores, V, scale, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    for fused in (True, False):
        out = csa.attention_pipeline(rp, ci, dev(Q), dev(K), dev(V), scale=scale, fused=fused)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, f"fused={fused}")


# ---------------------------------------------------------------------------
# backward operations: transpose, value gather, softmax backward and the
# gradients of SpMM, SDDMM and the attention
# ---------------------------------------------------------------------------

def _graphs_for_backward():
    return {"skew": skew_graph(1), "dup": dup_graph(3), "short": short_rows_graph(503),
            "edges": chunk_edge_graph(504)}


@pytest.mark.parametrize("graph", ["skew", "dup", "short", "edges", "empty"])
def test_transpose_bit_exact(graph):
    if graph == "empty":
        csr = CSR(5, 7, np.zeros(6, np.int32), np.zeros(0, np.int32))
    else:
        csr = _graphs_for_backward()[graph]
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    want = oracle.transpose(csr.row_ptr, csr.col_idx, csr.n_cols)
    for got, exp, name in zip(t, want, ("row_ptr", "col_idx", "perm")):
        assert np.array_equal(got.cpu().numpy(), exp), name
    # values follow their entries
    vals = np.random.default_rng(5).standard_normal(csr.nnz).astype(np.float32)
    if csr.nnz:
        got = csa.gather_values(t.perm, dev(vals)).cpu().numpy()
        assert np.array_equal(got, vals[want[2]])


@pytest.mark.gpu
def test_transpose_rows_in_range_for_unvalidated_row_ptr():
    # A row_ptr that is not monotone (and not checked: no validation flag)
    # still gives every transposed entry a row index inside [0, n_rows) and a
    # permutation of the entries, so later products never index out of range.
    n_rows, nnz = 6, 40
    rp = np.array([0, 25, 3, 31, 12, 50, 40], np.int32)  # 50 > nnz is clamped
    ci = np.random.default_rng(77).integers(0, 9, nnz).astype(np.int32)
    t = csa.transpose(dev(rp), dev(ci), 9)
    rows = t.col_idx.cpu().numpy()
    assert rows.min() >= 0 and rows.max() < n_rows
    assert np.array_equal(np.sort(t.perm.cpu().numpy()), np.arange(nnz))
    # each entry lies in the clamped range of the row it was given (ranges of
    # such a row_ptr overlap, so which of the covering rows is not fixed)
    bounds = np.clip(rp, 0, nnz)
    bounds[0], bounds[-1] = 0, nnz
    entry = t.perm.cpu().numpy()
    assert np.all((bounds[rows] <= entry) & (entry < bounds[rows + 1]))


def _probs_and_grad(csr, seed, scale):
    rng = np.random.default_rng(seed)
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    zero = np.zeros((csr.n_cols, 1), np.float32)
    p = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, scale, want_probs=True,
                         threads=oracle.default_threads())[2].astype(np.float32)
    g = rng.standard_normal(csr.nnz).astype(np.float32)
    return p, g


@pytest.mark.parametrize("graph", ["skew", "short", "edges"])
@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_row_softmax_backward_every_schedule(graph, scale):
    csr = _graphs_for_backward()[graph]
    p, g = _probs_and_grad(csr, 600, scale)
    ref, mag = oracle.softmax_backward(csr.row_ptr, p, g, scale, threads=oracle.default_threads())
    rp, pd, gd = dev(csr.row_ptr), dev(p), dev(g)
    prob, _ = csa.make_problem("row_softmax_backward", rp, None, pd, gd, scale=scale)
    scheds = csa.candidates(prob)
    assert {s.chunk_items for s in scheds} == {256, 512}
    for s in scheds:
        out = csa.row_softmax_backward(rp, pd, gd, scale=scale, schedule=s).cpu().numpy()
        assert_close(out, ref, mag, TOL_F32, sched_id(s))
    out = csa.row_softmax_backward(rp, pd, gd, scale=scale).cpu().numpy()  # automatic selection
    assert_close(out, ref, mag, TOL_F32, "auto")
    x = dev(g)
    csa.row_softmax_backward(rp, pd, x, scale=scale, out=x)  # in place over the gradient
    assert_close(x.cpu().numpy(), ref, mag, TOL_F32, "in place")


@pytest.mark.parametrize("graph", ["skew", "dup"])
def test_spmm_backward(graph):
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(610)
    F = 24
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dY = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    dvals, dX = csa.spmm_backward(rp, ci, dev(vals), dev(X), dev(dY))
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, dY, X, threads=oracle.default_threads())
    assert_close(dvals.cpu().numpy(), ref, mag, TOL_F32, "d vals")
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, vals.astype(np.float64), dY, csr.n_cols)
    assert_close(dX.cpu().numpy(), ref, mag, TOL_F32, "dX")
    # no edge values: A = pattern of ones, no value gradient
    dv0, dX1 = csa.spmm_backward(rp, ci, None, dev(X), dev(dY))
    assert dv0 is None
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, None, dY, csr.n_cols)
    assert_close(dX1.cpu().numpy(), ref, mag, TOL_F32, "dX, unit values")


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("F,dt", [(3, "f32"), (24, "f32"), (130, "f32"), (64, "bf16")])
def test_spmm_perm_every_schedule(graph, F, dt):
    """A^T X with A's values read through the transposed pattern's perm
    (csr_spmm_perm) under every schedule: against the oracle's transpose
    product, and bit for bit equal to the same schedule over the values
    gathered into the transposed order."""
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(615)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    Xf = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    if dt == "bf16":
        Xb = to_bf16_bits(Xf)
        Xd, Xref, tol = bf16_dev(Xb), oracle.bf16_to_f32(Xb), TOL_BF16
    else:
        Xd, Xref, tol = dev(Xf), Xf, TOL_F32
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    vd = dev(vals)
    vt = csa.gather_values(t.perm, vd)
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, vals.astype(np.float64), Xref, csr.n_cols)
    prob, _ = csa.make_problem("spmm", t.row_ptr, t.col_idx, vt, Xd)
    for s in schedules(prob):
        got = csa.spmm(t.row_ptr, t.col_idx, vd, Xd, val_idx=t.perm, schedule=s)
        e = assert_close(got.cpu().numpy(), ref, mag, tol, sched_id(s))
        assert e <= TOL_F32, sched_id(s)
        want = csa.spmm(t.row_ptr, t.col_idx, vt, Xd, schedule=s)
        assert torch.equal(got, want), sched_id(s)
    got = csa.spmm_transposed(t, vd, Xd)  # automatic selection
    assert_close(got.cpu().numpy(), ref, mag, tol, "auto")


def test_spmm_perm_errors_and_validation():
    csr = skew_graph(3, n_rows=600, n_cols=4000, giant=3000)
    rng = np.random.default_rng(616)
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    vd = dev(rng.standard_normal(csr.nnz).astype(np.float32))
    X = dev(rng.standard_normal((csr.n_rows, 16)).astype(np.float32))
    with pytest.raises(ValueError):
        csa.spmm(t.row_ptr, t.col_idx, None, X, val_idx=t.perm)
    with pytest.raises(ValueError):
        csa.spmm(t.row_ptr, t.col_idx, vd, X, val_idx=t.perm[1:])
    lib = csa.load_library()
    ctx = csa.Context(0, None)
    Y = torch.empty((csr.n_cols, 16), device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.csr_spmm_perm(ctx.handle, csr.n_cols, csr.n_rows, csr.nnz, t.row_ptr.data_ptr(), t.col_idx.data_ptr(),
                           vd.data_ptr(), None, X.data_ptr(), 0, 16, 16, Y.data_ptr(), 16, None, ws.data_ptr(),
                           ws.numel(), st)
    assert rc == -1  # CSR_ERR_NULL
    ctx.close()
    # an index out of range is caught on a validating context, before any product runs
    vctx = csa.Context(0, None, csa.CTX_VALIDATE)
    for badv in (csr.nnz, -1):
        bad = t.perm.clone()
        bad[csr.nnz // 2] = badv
        with pytest.raises(csa.CsrError) as ei:
            csa.spmm(t.row_ptr, t.col_idx, vd, X, val_idx=bad, ctx=vctx)
        assert "CSR_ERR_INVALID_CSR" in str(ei.value)
    ref = csa.spmm_transposed(t, vd, X, fused=False)
    got = csa.spmm_transposed(t, vd, X, ctx=vctx)
    assert torch.allclose(got, ref, rtol=1e-5, atol=1e-5)
    vctx.close()


def test_sddmm_backward():
    csr = skew_graph(7, n_rows=1200, n_cols=9000, giant=5000)
    rng = np.random.default_rng(620)
    K = 20
    U = rng.standard_normal((csr.n_rows, K)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, K)).astype(np.float32)
    g = rng.standard_normal(csr.nnz).astype(np.float32)
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    dU, dV = csa.sddmm_backward(rp, ci, dev(U), dev(V), dev(g), transposed=t)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, g, V, threads=oracle.default_threads())
    assert_close(dU.cpu().numpy(), ref, mag, TOL_F32, "dU")
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, g.astype(np.float64), U, csr.n_cols)
    assert_close(dV.cpu().numpy(), ref, mag, TOL_F32, "dV")


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_attention_backward(graph, scale):
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(630)
    F = 16
    sc = (2 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    dS, dV = csa.attention_backward(rp, ci, dev(sc), dev(V), dev(dO), scale=scale)
    ref, mag = oracle.attention_backward_scores(csr.row_ptr, csr.col_idx, sc, V, dO, scale,
                                                threads=oracle.default_threads())
    assert_close(dS.cpu().numpy(), ref, mag, TOL_F32, "d scores")
    zero = np.zeros((csr.n_cols, 1), np.float32)
    P = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, scale, want_probs=True)[2]
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, P, dO, csr.n_cols)
    assert_close(dV.cpu().numpy(), ref, mag, TOL_F32, "dV")


def test_backward_edge_cases():
    # no entries at all: nothing to write, shapes still right
    rp = dev(np.zeros(6, np.int32))
    ci = dev(np.zeros(0, np.int32))
    empty = dev(np.zeros(0, np.float32))
    assert csa.row_softmax_backward(rp, empty, empty).numel() == 0
    t = csa.transpose(rp, ci, 0)
    assert t.row_ptr.cpu().numpy().tolist() == [0] and t.col_idx.numel() == 0
    assert csa.gather_values(t.perm, empty).numel() == 0
    # a single entry per row: the softmax is 1, its gradient 0
    csr = CSR(4, 3, np.arange(5, dtype=np.int32), np.array([2, 0, 1, 2], np.int32))
    rp, ci = pattern_dev(csr)
    p = dev(np.ones(4, np.float32))
    g = dev(np.array([3.0, -1.0, 0.5, 7.0], np.float32))
    assert np.array_equal(csa.row_softmax_backward(rp, p, g, scale=0.5).cpu().numpy(), np.zeros(4, np.float32))
    # the gradient of an identity-pattern attention with respect to V is dOut itself (bit-exact: p = 1)
    n = 300
    csr = CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32))
    rp, ci = pattern_dev(csr)
    rng = np.random.default_rng(640)
    dO = rng.standard_normal((n, 8)).astype(np.float32)
    dS, dV = csa.attention_backward(rp, ci, dev(rng.standard_normal(n).astype(np.float32)),
                                    dev(rng.standard_normal((n, 8)).astype(np.float32)), dev(dO))
    assert np.array_equal(dV.cpu().numpy(), dO)
    assert np.array_equal(dS.cpu().numpy(), np.zeros(n, np.float32))


def test_backward_deterministic():
    csr = skew_graph(9, n_rows=1500, n_cols=8000, giant=6000)
    rng = np.random.default_rng(650)
    sc = dev(rng.standard_normal(csr.nnz).astype(np.float32))
    V = dev(rng.standard_normal((csr.n_cols, 12)).astype(np.float32))
    dO = dev(rng.standard_normal((csr.n_rows, 12)).astype(np.float32))
    rp, ci = pattern_dev(csr)
    a = [x.cpu().numpy() for x in csa.attention_backward(rp, ci, sc, V, dO, scale=0.3)]
    b = [x.cpu().numpy() for x in csa.attention_backward(rp, ci, sc, V, dO, scale=0.3)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# column-part segment format
# ---------------------------------------------------------------------------

def _format_graph(name):
    if name == "skew":
        return skew_graph(1)
    if name == "dup":
        return dup_graph(3)
    if name == "short":
        return short_rows_graph(5)
    if name == "edges":
        return chunk_edge_graph(6)
    if name == "empty":
        return CSR(50, 40, np.zeros(51, np.int32), np.zeros(0, np.int32))
    raise KeyError(name)


@pytest.mark.parametrize("graph", ["skew", "dup", "short", "edges", "empty"])
@pytest.mark.parametrize("P,T", [(1, 0), (4, 0), (32, 0), (256, 0), (8, 4), (32, 300)])
def test_hybrid_format_bit_exact(graph, P, T):
    csr = _format_graph(graph)
    rp, ci = pattern_dev(csr)
    h = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)
    want = oracle.hybrid_format(csr.row_ptr, csr.col_idx, csr.n_cols, P, whole_below=T)
    assert h.part_cols == want["part_cols"] and h.n_seg == len(want["seg_row"])
    for k in ("perm", "col_idx", "seg_ptr", "seg_row", "row_seg_ptr", "row_seg"):
        assert np.array_equal(getattr(h, k).cpu().numpy(), want[k]), k
    h2 = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)  # rebuilt: the same arrays
    for k in ("perm", "seg_ptr", "row_seg"):
        assert torch.equal(getattr(h, k), getattr(h2, k))


# F = 300: one segment per wave in the row-group mapping (64 lanes, 2 passes of 4)
@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("F", [1, 4, 32, 100, 300])
def test_hybrid_spmm_every_schedule(graph, F):
    csr = _format_graph(graph)
    rng = np.random.default_rng(1100 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    Xd = dev(X)
    for P, T in ((2, 0), (8, 0), (32, 0), (128, 0), (8, 40), (32, 300)):
        h = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)
        hv = csa.hybrid_values(h, dev(vals))
        p = csa.hybrid_problem(h, "spmm", hv, Xd)
        for s in schedules(p, thorough=(P == 8 and T == 0 and graph == "skew")):
            Y = csa.hybrid_spmm(h, hv, Xd, schedule=s)
            assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, f"P{P}-T{T}-" + sched_id(s))
        Y = csa.hybrid_spmm(h, hv, Xd)  # selected
        assert_close(Y.cpu().numpy(), ref, mag, TOL_F32, f"P{P}-T{T}-auto")
    ones, omag = oracle.spmm(csr.row_ptr, csr.col_idx, None, X, threads=oracle.default_threads())
    Y = csa.hybrid_spmm(h, None, Xd)
    assert_close(Y.cpu().numpy(), ones, omag, TOL_F32, "unit values")


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("K", [1, 4, 32, 128])
def test_hybrid_sddmm_every_schedule(graph, K):
    csr = _format_graph(graph)
    rng = np.random.default_rng(1200 + K)
    U = rng.standard_normal((csr.n_rows, K)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, K)).astype(np.float32)
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    Ud, Vd = dev(U), dev(V)
    for P, T in ((2, 0), (8, 0), (32, 0), (32, 300)):
        h = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)
        p = csa.hybrid_problem(h, "sddmm", Ud, Vd)
        for s in schedules(p, thorough=(P == 8 and graph == "skew")):
            out = csa.hybrid_sddmm(h, Ud, Vd, schedule=s)
            assert_close(out.cpu().numpy(), ref, mag, TOL_F32, f"P{P}-" + sched_id(s))
        out = csa.hybrid_sddmm(h, Ud, Vd)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, f"P{P}-auto")


def test_hybrid_edge_cases():
    # no entries: Y is +0 everywhere, SDDMM writes nothing
    csr = _format_graph("empty")
    rp, ci = pattern_dev(csr)
    h = csa.hybrid_format(rp, ci, csr.n_cols, 8)
    assert h.n_seg == 0 and h.row_seg_ptr.cpu().numpy().tolist() == [0] * 51
    Y = csa.hybrid_spmm(h, None, dev(np.ones((40, 6), np.float32))).cpu().numpy()
    assert np.all(Y == 0) and not np.signbit(Y).any()
    out = csa.hybrid_sddmm(h, dev(np.ones((50, 6), np.float32)), dev(np.ones((40, 6), np.float32)))
    assert out.numel() == 0
    # fewer columns than parts, strided operands, empty rows stay +0
    rng = np.random.default_rng(41)
    csr = graphs.random_small_graph(2000, 3, 0.5, rng, empty_frac=0.3, allow_dup=True)
    rp, ci = pattern_dev(csr)
    h = csa.hybrid_format(rp, ci, 3, 32)
    assert h.part_cols == 1
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((3, 20)).astype(np.float32)
    Xs = torch.zeros((3, 24), device="cuda")
    Xs[:, :20] = dev(X)
    Ys = torch.full((2000, 28), 7.0, device="cuda")
    csa.hybrid_spmm(h, csa.hybrid_values(h, dev(vals)), Xs[:, :20], out=Ys[:, :20])
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X)
    Y = Ys.cpu().numpy()
    assert_close(Y[:, :20], ref, mag, TOL_F32, "strided")
    assert np.all(Y[:, 20:] == 7.0)  # the padding columns are not written
    empty = np.diff(csr.row_ptr) == 0
    assert np.all(Y[empty, :20] == 0) and not np.signbit(Y[empty, :20]).any()


def test_hybrid_deterministic_and_errors():
    csr = skew_graph(4, n_rows=2000, n_cols=40_000, giant=20_000)
    rng = np.random.default_rng(9)
    rp, ci = pattern_dev(csr)
    h = csa.hybrid_format(rp, ci, csr.n_cols, 16)
    hv = csa.hybrid_values(h, dev(rng.standard_normal(csr.nnz).astype(np.float32)))
    X = dev(rng.standard_normal((csr.n_cols, 16)).astype(np.float32))
    U = dev(rng.standard_normal((csr.n_rows, 16)).astype(np.float32))
    assert torch.equal(csa.hybrid_spmm(h, hv, X), csa.hybrid_spmm(h, hv, X))
    assert torch.equal(csa.hybrid_sddmm(h, U, X), csa.hybrid_sddmm(h, U, X))
    # selection: replayed from the cache, and the schedule the call itself uses
    ctx = csa.Context(0, None)
    for op, a, b in (("spmm", hv, X), ("sddmm", U, X)):
        s1, sig1 = csa.hybrid_select(h, op, a, b, ctx=ctx)
        s2, sig2 = csa.hybrid_select(h, op, a, b, mode="replay", ctx=ctx)
        assert bytes(s1) == bytes(s2) and sig1 == sig2 and sig1 != 0
        run = csa.hybrid_spmm if op == "spmm" else csa.hybrid_sddmm
        assert torch.equal(run(h, a, b, schedule=s1, ctx=ctx), run(h, a, b, ctx=ctx))
    assert ctx.cache_info()["entries"] == 2
    ctx.close()
    lib = csa.load_library()
    ctx = csa.default_context(0)
    st = torch.cuda.current_stream().cuda_stream
    n = ctypes.c_int64()
    assert lib.csr_hybrid_capacity(10, 100, 3, ctypes.byref(n)) == -2
    assert lib.csr_hybrid_capacity(10, 100, 512, ctypes.byref(n)) == -2
    assert lib.csr_hybrid_capacity(10, 100, 4, ctypes.byref(n)) == 0 and n.value == 40
    # segment capacity below the bound
    d = _ffi.CsrHybrid.from_buffer_copy(bytes(h.desc))
    d.seg_cap = h.desc.seg_cap - 1
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    assert lib.csr_hybrid_build(ctx.handle, rp.data_ptr(), ci.data_ptr(), ctypes.byref(d), ws.data_ptr(),
                                ws.numel(), st) == -5
    # a description that was never built
    d = _ffi.CsrHybrid.from_buffer_copy(bytes(h.desc))
    d.whole_below = -1
    assert lib.csr_hybrid_build(ctx.handle, rp.data_ptr(), ci.data_ptr(), ctypes.byref(d), ws.data_ptr(),
                                ws.numel(), st) == -2
    d = _ffi.CsrHybrid.from_buffer_copy(bytes(h.desc))
    d.n_seg = -1
    Y = torch.empty((csr.n_rows, 16), device="cuda")
    assert lib.csr_hybrid_spmm(ctx.handle, ctypes.byref(d), hv.data_ptr(), X.data_ptr(), 0, 16, 16, Y.data_ptr(), 16,
                               None, ws.data_ptr(), ws.numel(), st) == -2
    # workspace too small, ldy below the width
    assert lib.csr_hybrid_spmm(ctx.handle, ctypes.byref(h.desc), hv.data_ptr(), X.data_ptr(), 0, 16, 16, Y.data_ptr(),
                               16, None, ws.data_ptr(), 4096, st) == -5
    assert lib.csr_hybrid_spmm(ctx.handle, ctypes.byref(h.desc), hv.data_ptr(), X.data_ptr(), 0, 16, 16, Y.data_ptr(),
                               8, None, ws.data_ptr(), ws.numel(), st) == -2
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# HIP graph capture of launch-bound calls
# ---------------------------------------------------------------------------

def test_graph_capture_replays_match_eager():
    """With explicit schedules (and no validation) the calls only enqueue
    kernels: captured into a graph, every replay, with eager work and
    synchronisations between the replays, equals the eager result bit for bit."""
    c = __import__("synth").configs.make_config("c1")
    csr = c["csr"]
    rp, ci = pattern_dev(csr)
    S, V = dev(c["scores"]), dev(c["V"])
    rng = np.random.default_rng(3)
    X = dev(rng.standard_normal((csr.n_cols, 32)).astype(np.float32))
    outs = {"att": torch.empty((csr.n_rows, V.shape[1]), device="cuda"),
            "spmm": torch.empty((csr.n_rows, 32), device="cuda"),
            "sddmm": torch.empty(csr.nnz, device="cuda"),
            "fmt": torch.empty((csr.n_rows, 32), device="cuda")}
    sa, _ = csa.select("attention", rp, ci, S, V, out=outs["att"])
    ss, _ = csa.select("spmm", rp, ci, S, X, out=outs["spmm"])
    sd, _ = csa.select("sddmm", rp, ci, X, X, out=outs["sddmm"])
    h = csa.hybrid_format(rp, ci, csr.n_cols, 4, whole_below=8)
    hv = csa.hybrid_values(h, S)
    sh, _ = csa.hybrid_select(h, "spmm", hv, X)

    def step():
        csa.attention(rp, ci, S, V, out=outs["att"], schedule=sa)
        csa.spmm(rp, ci, S, X, out=outs["spmm"], schedule=ss)
        csa.sddmm(rp, ci, X, X, out=outs["sddmm"], schedule=sd)
        csa.hybrid_spmm(h, hv, X, out=outs["fmt"], schedule=sh)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream, as graph capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for v in outs.values():
            v.fill_(float("nan"))
        # eager work between the replays (other inputs, other outputs)
        csa.spmm(rp, ci, None, X * (r + 2))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], eager[k]), (r, k)
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, c["scores"], c["V"])
    assert_close(outs["att"].cpu().numpy(), ref, mag, TOL_F32, "graph attention")


@pytest.mark.parametrize("F", [4, 5, 6, 7, 255, 257, 602, 1021, 2600, 4096])
def test_wide_lanes_misaligned_operands(F):
    # 4 floats per lane over rows that are only 4-byte aligned: X and Y are
    # column views at an odd offset of wider buffers (odd leading dimensions),
    # every remainder of F mod 4 and the 1, 2, 4, 12 and 16 pass layouts
    # (a width above 1024 needs 16-byte aligned rows to be a valid problem:
    # there the views start 4 floats in)
    o = 1 if F <= 1024 else 4
    csr = skew_graph(11, n_rows=700, n_cols=3000, giant=2500)
    rng = np.random.default_rng(1200 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    Xb = rng.standard_normal((csr.n_cols, F + 2 * o)).astype(np.float32)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, Xb[:, o:F + o], threads=oracle.default_threads())
    rp, ci = pattern_dev(csr)
    Xd = dev(Xb)[:, o:F + o]
    Yd = torch.full((csr.n_rows, F + 4 * o), float("nan"), device="cuda")
    Y = Yd[:, 3 * o:F + 3 * o]
    p, _ = csa.make_problem("spmm", rp, ci, dev(vals), Xd, out=Y)
    s = csa.CsrSchedule.from_buffer_copy(bytes(csa.default_schedule(p)))
    s.mapping, s.vec, s.group_lanes, s.chunk_items, s.long_row = csa.MAP_ROWGROUP, 4, 64, 0, 0
    s.passes = min(v for v in (1, 2, 3, 4, 5, 6, 8, 12, 16) if v * 256 >= F)
    s.flags = csa.SCHED_WIDE
    csa.spmm(rp, ci, dev(vals), Xd, out=Y, schedule=s)
    torch.cuda.synchronize()
    got = Yd.cpu().numpy()
    assert_close(got[:, 3 * o:F + 3 * o], ref, mag, TOL_F32, f"wide F{F}")
    assert np.isnan(got[:, :3 * o]).all() and np.isnan(got[:, F + 3 * o:]).all()  # nothing written outside Y
    ones, omag = oracle.spmm(csr.row_ptr, csr.col_idx, None, Xb[:, o:F + o], threads=oracle.default_threads())
    csa.spmm(rp, ci, None, Xd, out=Y, schedule=s)
    assert_close(Y.cpu().numpy(), ones, omag, TOL_F32, f"wide F{F} unit values")
    # over the format (partial rows with leading dimension F, then the sum)
    h = csa.hybrid_format(rp, ci, csr.n_cols, 8, whole_below=16)
    hv = csa.hybrid_values(h, dev(vals))
    Yh = csa.hybrid_spmm(h, hv, Xd, schedule=s)
    assert_close(Yh.cpu().numpy(), ref, mag, TOL_F32, f"wide F{F} over the format")


@pytest.mark.parametrize("F", [4, 602])
def test_infinite_features_propagate_without_nan(F):
    # X row 7 holds +inf in feature 0: every row with an entry in column 7
    # (positive weights) gets +inf there and stays finite elsewhere; rows of
    # 1-3 entries leave padded slots in the last batch of every mapping, which
    # must add nothing (0 * inf would be NaN)
    rng = np.random.default_rng(77 + F)
    n_rows, n_cols = 300, 50
    deg = rng.integers(0, 9, n_rows)
    cols = [np.sort(rng.choice(n_cols, d, replace=False)) for d in deg]
    for r in range(0, n_rows, 5):  # many rows start with column 7
        if deg[r] > 0:
            cols[r][0] = 7
            cols[r] = np.sort(cols[r])
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    col_idx = np.concatenate(cols).astype(np.int32)
    vals = rng.uniform(0.5, 1.5, col_idx.size).astype(np.float32)
    X = rng.standard_normal((n_cols, F)).astype(np.float32)
    X[7, 0] = np.inf
    csr = CSR(n_rows, n_cols, row_ptr, col_idx)
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=1)
    rp, ci = pattern_dev(csr)
    p, _ = csa.make_problem("spmm", rp, ci, dev(vals), dev(X))
    has7 = np.array([7 in c for c in cols])
    assert has7.sum() > 20
    for s in schedules(p):
        Y = csa.spmm(rp, ci, dev(vals), dev(X), schedule=s).cpu().numpy()
        assert not np.isnan(Y).any(), sched_id(s)
        assert np.isposinf(Y[has7, 0]).all() and np.isfinite(Y[~has7]).all(), sched_id(s)
        fin = np.isfinite(ref)
        assert_close(np.where(fin, Y, 0), np.where(fin, ref, 0), np.where(fin, mag, 1), TOL_F32, sched_id(s))


# ---------------------------------------------------------------------------
# several heads of given scores (head-major [H, nnz]): each head against the
# oracle's one-head attention, probabilities [nnz, H]
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("H,D,dt", [(2, 16, "f32"), (3, 4, "f32"), (8, 64, "f32"), (4, 32, "bf16")])
def test_attention_heads_given_scores(graph, H, D, dt):
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(700 + H * D)
    scores = (2 * rng.standard_normal((H, csr.nnz))).astype(np.float32)
    Vf = rng.standard_normal((csr.n_cols, H, D)).astype(np.float32)
    if dt == "bf16":
        Vb = to_bf16_bits(Vf)
        Vd, Vref, tol = bf16_dev(Vb), oracle.bf16_to_f32(Vb), TOL_BF16
    else:
        Vd, Vref, tol = dev(Vf), Vf, TOL_F32
    rp, ci = pattern_dev(csr)
    sd = dev(scores)
    scale = 0.37
    refs = [oracle.attention(csr.row_ptr, csr.col_idx, scores[h], np.ascontiguousarray(Vref[:, h, :]), scale,
                             want_probs=True, threads=oracle.default_threads()) for h in range(H)]
    probs = torch.empty((csr.nnz, H), device="cuda")
    out = csa.attention(rp, ci, sd, Vd, scale=scale, probs=probs)
    assert tuple(out.shape) == (csr.n_rows, H, D)
    got, gp = out.cpu().numpy(), probs.cpu().numpy()
    for h, (ref, mag, pref) in enumerate(refs):
        e = assert_close(got[:, h, :], ref, mag, tol, f"head {h}")
        assert e <= TOL_F32, (h, e)
        live = pref > 0
        assert np.all(gp[~live, h] == 0)
        assert float(np.max(np.abs(gp[live, h] - pref[live]) / pref[live], initial=0.0)) <= 1e-5, h
    # the schedule the heads share, given explicitly: the same results bit for bit
    p, _ = csa.make_problem("attention", rp, ci, sd[0], Vd.view(csr.n_cols, H * D)[:, :D], scale=scale)
    for s in schedules(p, thorough=False):
        o2 = csa.attention(rp, ci, sd, Vd, scale=scale, schedule=s).cpu().numpy()
        for h, (ref, mag, _) in enumerate(refs):
            assert_close(o2[:, h, :], ref, mag, tol, f"head {h} {sched_id(s)}")


def test_attention_heads_given_scores_errors():
    csr = dup_graph(3)
    rp, ci = pattern_dev(csr)
    sd = dev(np.zeros((2, csr.nnz), np.float32))
    V = dev(np.zeros((csr.n_cols, 2, 8), np.float32))
    with pytest.raises(ValueError):
        csa.attention(rp, ci, sd[:, 1:], V)  # scores of the wrong length
    with pytest.raises(ValueError):
        csa.attention(rp, ci, sd, dev(np.zeros((csr.n_cols, 3, 8), np.float32)))  # head counts differ
    with pytest.raises(ValueError):
        csa.attention(rp, ci, sd, V, out=torch.empty((csr.n_rows, 2, 4), device="cuda"))
    with pytest.raises(ValueError):
        csa.attention(rp, ci, sd, V, probs=torch.empty((2, csr.nnz), device="cuda"))  # probs are [nnz, H]


# ---------------------------------------------------------------------------
# SpMM + SDDMM sharing the gathered rows (csr_spmm_sddmm)
# ---------------------------------------------------------------------------

def _as_op(s, op):
    t = csa.CsrSchedule.from_buffer_copy(bytes(s))
    t.op = op
    return t


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("F", [1, 5, 32, 64, 100])
def test_spmm_sddmm_every_schedule(graph, F):
    """Y = A X and z_e = <U[row_e], X[col_e]> from one pass under every
    schedule: each against the oracle's SpMM and SDDMM, and bit for bit equal
    to csr_spmm and csr_sddmm under the same lane layout and mapping (the same
    sums in the same order)."""
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(640 + F)
    vals = rng.standard_normal(csr.nnz).astype(np.float32)
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    U = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    vd, Xd, Ud = dev(vals), dev(X), dev(U)
    th = oracle.default_threads()
    refY, magY = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=th)
    refZ, magZ = oracle.sddmm(csr.row_ptr, csr.col_idx, U, X, threads=th)
    p, _ = csa.make_problem("spmm_sddmm", rp, ci, vd, Xd, Ud)
    scheds = schedules(p)
    assert any(s.mapping == csa.MAP_ROWGROUP for s in scheds) and any(s.mapping == csa.MAP_MERGEPATH for s in scheds)
    for s in scheds:
        Y, z = csa.spmm_sddmm(rp, ci, vd, Xd, Ud, schedule=s)
        assert_close(Y.cpu().numpy(), refY, magY, TOL_F32, f"Y {sched_id(s)}")
        assert_close(z.cpu().numpy(), refZ, magZ, TOL_F32, f"z {sched_id(s)}")
        assert torch.equal(Y, csa.spmm(rp, ci, vd, Xd, schedule=_as_op(s, _ffi.OP_SPMM))), sched_id(s)
        assert torch.equal(z, csa.sddmm(rp, ci, Ud, Xd, schedule=_as_op(s, _ffi.OP_SDDMM))), sched_id(s)
    # without values (all ones), automatic selection
    refY1, magY1 = oracle.spmm(csr.row_ptr, csr.col_idx, np.ones(csr.nnz, np.float32), X, threads=th)
    Y, z = csa.spmm_sddmm(rp, ci, None, Xd, Ud)
    assert_close(Y.cpu().numpy(), refY1, magY1, TOL_F32, "ones")
    assert_close(z.cpu().numpy(), refZ, magZ, TOL_F32, "ones z")


@pytest.mark.parametrize("graph", ["skew", "dup", "short", "edges"])
@pytest.mark.parametrize("F", [24, 64])
def test_spmm_sddmm_transposed(graph, F):
    """On A^T with A's values read and z written through the transposed
    pattern's perm: dV = P^T dOut and dP = dOut V^T at A's entry positions
    (the two products of attention's backward that gather dOut)."""
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(650 + F)
    P = rng.random(csr.nnz).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    Pd, dOd, Vd = dev(P), dev(dO), dev(V)
    refV, magV = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, P.astype(np.float64), dO, csr.n_cols)
    refP, magP = oracle.sddmm(csr.row_ptr, csr.col_idx, dO, V, threads=oracle.default_threads())
    p, _ = csa.make_problem("spmm_sddmm", t.row_ptr, t.col_idx, Pd, dOd, Vd, val_idx=t.perm)
    for s in schedules(p) + [None]:
        dV, dP = csa.spmm_sddmm(t.row_ptr, t.col_idx, Pd, dOd, Vd, val_idx=t.perm, z_idx=t.perm, schedule=s)
        what = "auto" if s is None else sched_id(s)
        assert_close(dV.cpu().numpy(), refV, magV, TOL_F32, f"dV {what}")
        assert_close(dP.cpu().numpy(), refP, magP, TOL_F32, f"dP {what}")


def test_spmm_sddmm_infinite_features():
    """An infinite feature gives an infinite dot product, not NaN, also where
    lanes past the width (F = 5 on 8 lanes) read the row's first features."""
    csr = dup_graph(11)
    rng = np.random.default_rng(660)
    F = 5
    X = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    U = (rng.random((csr.n_rows, F)) + 0.5).astype(np.float32)
    X[::7, 0] = np.inf
    rp, ci = pattern_dev(csr)
    vd = dev(np.ones(csr.nnz, np.float32))
    p, _ = csa.make_problem("spmm_sddmm", rp, ci, vd, dev(X), dev(U))
    want = np.where(np.isin(csr.col_idx, np.arange(0, csr.n_cols, 7)), np.inf, 0.0)
    for s in schedules(p, thorough=False):
        _, z = csa.spmm_sddmm(rp, ci, vd, dev(X), dev(U), schedule=s)
        z = z.cpu().numpy()
        hot = want == np.inf
        assert np.all(z[hot] == np.inf), sched_id(s)
        assert np.all(np.isfinite(z[~hot])), sched_id(s)


def test_spmm_sddmm_errors_and_validation():
    csr = skew_graph(3, n_rows=600, n_cols=4000, giant=3000)
    rng = np.random.default_rng(661)
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols)
    vd = dev(rng.standard_normal(csr.nnz).astype(np.float32))
    X = dev(rng.standard_normal((csr.n_rows, 16)).astype(np.float32))
    U = dev(rng.standard_normal((csr.n_cols, 16)).astype(np.float32))
    with pytest.raises(ValueError):
        csa.spmm_sddmm(t.row_ptr, t.col_idx, None, X, U, val_idx=t.perm)
    with pytest.raises(ValueError):
        csa.spmm_sddmm(t.row_ptr, t.col_idx, vd, X, U[1:])
    with pytest.raises(ValueError):
        csa.spmm_sddmm(t.row_ptr, t.col_idx, vd, X, U, z=torch.empty(csr.nnz - 1, device="cuda"))
    with pytest.raises(TypeError):
        csa.spmm_sddmm(t.row_ptr, t.col_idx, vd, X.to(torch.bfloat16), U)
    lib = csa.load_library()
    ctx = csa.Context(0, None)
    Y = torch.empty((csr.n_cols, 16), device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.csr_spmm_sddmm(ctx.handle, csr.n_cols, csr.n_rows, csr.nnz, t.row_ptr.data_ptr(), t.col_idx.data_ptr(),
                            vd.data_ptr(), None, X.data_ptr(), 16, 16, U.data_ptr(), 16, Y.data_ptr(), 16, None,
                            None, None, ws.data_ptr(), ws.numel(), st)
    assert rc == -1  # CSR_ERR_NULL: no z
    ctx.close()
    # an index out of range is caught on a validating context, before any product runs
    vctx = csa.Context(0, None, csa.CTX_VALIDATE)
    for which in ("val_idx", "z_idx"):
        bad = t.perm.clone()
        bad[csr.nnz // 2] = csr.nnz
        kw = {"val_idx": t.perm, "z_idx": t.perm, which: bad}
        with pytest.raises(csa.CsrError) as ei:
            csa.spmm_sddmm(t.row_ptr, t.col_idx, vd, X, U, ctx=vctx, **kw)
        assert "CSR_ERR_INVALID_CSR" in str(ei.value)
    vctx.close()


# ---------------------------------------------------------------------------
# the inverse permutation (entries of A to their positions in A^T)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("graph", ["skew", "dup", "short", "edges"])
def test_inverse_permutation_bit_exact(graph):
    csr = _graphs_for_backward()[graph]
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols, inverse=True)
    perm = oracle.transpose(csr.row_ptr, csr.col_idx, csr.n_cols)[2]
    want = np.empty_like(perm)
    want[perm] = np.arange(perm.size, dtype=perm.dtype)
    assert np.array_equal(t.inv.cpu().numpy(), want)
    assert np.array_equal(csa.inverse_permutation(t.perm).cpu().numpy(), want)
    with pytest.raises(csa.CsrError):
        csa.inverse_permutation(t.perm, out=t.perm)  # perm and inv alias


def test_validating_context_row_softmax_ops():
    """The row softmax and its backward have no column indices: a validating
    context checks their row_ptr only (and still catches a bad one)."""
    csr = dup_graph(12)
    p, g = _probs_and_grad(csr, 602, 0.5)
    rp = dev(csr.row_ptr)
    sc = dev(np.random.default_rng(603).standard_normal(csr.nnz).astype(np.float32))
    vctx = csa.Context(0, None, csa.CTX_VALIDATE)
    s, _ = csa.select("row_softmax", rp, None, sc, scale=0.5, mode="estimate")
    assert torch.equal(csa.row_softmax(rp, sc, scale=0.5, ctx=vctx, schedule=s),
                       csa.row_softmax(rp, sc, scale=0.5, schedule=s))
    refb, mag = oracle.softmax_backward(csr.row_ptr, p, g, 0.5)
    got = csa.row_softmax_backward(rp, dev(p), dev(g), scale=0.5, ctx=vctx)
    assert_close(got.cpu().numpy(), refb, mag, TOL_F32, "validating context")
    bad = rp.clone()
    bad[5] = bad[6] + 1  # not monotone
    with pytest.raises(csa.CsrError) as ei:
        csa.row_softmax(bad, sc, scale=0.5, ctx=vctx)
    assert "CSR_ERR_INVALID_CSR" in str(ei.value)
    vctx.close()


@pytest.mark.parametrize("graph", ["skew", "dup", "short", "edges", "empty"])
@pytest.mark.parametrize("window_log2", [8, 12, 30])
def test_permutation_plan_bit_exact(graph, window_log2):
    """Two-pass permutations of a transposed pattern's perm and its inverse
    move per-entry values exactly as the direct gathers do, for windows from
    256 values (many groups) to 2^30 (one group)."""
    if graph == "empty":
        csr = CSR(5, 7, np.zeros(6, np.int32), np.zeros(0, np.int32))
    else:
        csr = _graphs_for_backward()[graph]
    rp, ci = pattern_dev(csr)
    t = csa.transpose(rp, ci, csr.n_cols, inverse=True)
    vals = dev(np.random.default_rng(670).standard_normal(csr.nnz).astype(np.float32))
    for q in (t.perm, t.inv):
        plan = csa.permutation_plan(q, window_log2=window_log2)
        got = csa.permute_values(plan, vals)
        want = vals.cpu().numpy()[q.cpu().numpy().astype(np.int64)]
        assert np.array_equal(got.cpu().numpy(), want)
        # the plan's arrays: q1 is q in window order, pos its inverse placement
        q1, pos = plan.q1.cpu().numpy(), plan.pos.cpu().numpy()
        assert np.array_equal(np.sort(pos), np.arange(csr.nnz))
        assert np.array_equal(q1[pos], q.cpu().numpy())
        win = q1.astype(np.int64) >> window_log2
        assert np.all(np.diff(win) >= 0)


def test_permutation_plan_errors():
    q = torch.arange(1000, dtype=torch.int32, device="cuda")
    with pytest.raises(csa.CsrError):
        csa.permutation_plan(q, window_log2=7)
    with pytest.raises(csa.CsrError):
        csa.permutation_plan(q, window_log2=31)
    plan = csa.permutation_plan(q)
    x = torch.ones(1000, device="cuda")
    with pytest.raises(csa.CsrError):
        csa.permute_values(plan, x, out=x)  # src and dst alias
    with pytest.raises(ValueError):
        csa.permute_values(plan, torch.ones(999, device="cuda"))


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
def test_attention_backward_through_plans(graph):
    """attention_backward over a transposed pattern with permutation plans
    (P into A^T's order and dP back in two passes) against the oracle, and
    equal to the index-based composition."""
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(671)
    F = 32
    sc = (2 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    tp = csa.transpose(rp, ci, csr.n_cols, plans=True)
    ti = csa.transpose(rp, ci, csr.n_cols, inverse=True)
    dS, dV = csa.attention_backward(rp, ci, dev(sc), dev(V), dev(dO), scale=0.5, transposed=tp)
    dS2, dV2 = csa.attention_backward(rp, ci, dev(sc), dev(V), dev(dO), scale=0.5, transposed=ti)
    assert torch.equal(dS, dS2) and torch.equal(dV, dV2)
    ref, mag = oracle.attention_backward_scores(csr.row_ptr, csr.col_idx, sc, V, dO, 0.5,
                                                threads=oracle.default_threads())
    assert_close(dS.cpu().numpy(), ref, mag, TOL_F32, "d scores")
    P = oracle.attention(csr.row_ptr, csr.col_idx, sc, np.zeros((csr.n_cols, 1), np.float32), 0.5,
                         want_probs=True)[2]
    refV, magV = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, P, dO, csr.n_cols)
    assert_close(dV.cpu().numpy(), refV, magV, TOL_F32, "dV")


def test_graph_capture_backward_step():
    """The attention backward step as library calls with explicit schedules
    (row softmax, P into A^T's order, the SpMM + SDDMM pass over A^T, dP back,
    softmax backward in place) captured into one graph: every replay, with
    eager work between the replays, equals the eager step bit for bit, and
    the gradients match the oracle."""
    csr = skew_graph(13, n_rows=1500, n_cols=20000, giant=8000)
    rng = np.random.default_rng(680)
    F, scale = 32, 0.5
    sc = (2 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    rp, ci = pattern_dev(csr)
    S, Vd, dOd = dev(sc), dev(V), dev(dO)
    t = csa.transpose(rp, ci, csr.n_cols, plans=True)
    e = lambda: torch.empty(csr.nnz, device="cuda")  # noqa: E731
    P, Pt, dPt, dP, tmp = e(), e(), e(), e(), e()
    dV = torch.empty((csr.n_cols, F), device="cuda")
    s_sm, _ = csa.select("row_softmax", rp, None, S, scale=scale, out=P)
    csa.row_softmax(rp, S, scale=scale, out=P, schedule=s_sm)
    csa.permute_values(t.to_t, P, out=Pt, tmp=tmp)
    s_d, _ = csa.select("spmm_sddmm", t.row_ptr, t.col_idx, Pt, dOd, Vd, out=dV)
    s_b, _ = csa.select("row_softmax_backward", rp, None, P, dP, scale=scale, out=dP)

    def step():
        csa.row_softmax(rp, S, scale=scale, out=P, schedule=s_sm)
        csa.permute_values(t.to_t, P, out=Pt, tmp=tmp)
        csa.spmm_sddmm(t.row_ptr, t.col_idx, Pt, dOd, Vd, out=dV, z=dPt, schedule=s_d)
        csa.permute_values(t.from_t, dPt, out=dP, tmp=tmp)
        csa.row_softmax_backward(rp, P, dP, scale=scale, out=dP, schedule=s_b)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream, as graph capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = (dP.clone(), dV.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        dP.fill_(float("nan"))
        dV.fill_(float("nan"))
        csa.spmm(rp, ci, None, Vd * (r + 2))  # eager work between the replays (V has the pattern's n_cols rows)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dP, eager[0]) and torch.equal(dV, eager[1]), r
    ref, mag = oracle.attention_backward_scores(csr.row_ptr, csr.col_idx, sc, V, dO, scale,
                                                threads=oracle.default_threads())
    assert_close(dP.cpu().numpy(), ref, mag, TOL_F32, "graph d scores")
    Pref = oracle.attention(csr.row_ptr, csr.col_idx, sc, np.zeros((csr.n_cols, 1), np.float32), scale,
                            want_probs=True)[2]
    refV, magV = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, Pref, dO, csr.n_cols)
    assert_close(dV.cpu().numpy(), refV, magV, TOL_F32, "graph dV")


@pytest.mark.parametrize("graph", ["skew", "dup", "edges"])
@pytest.mark.parametrize("D,F", [(32, 32), (16, 24)])
def test_attention_qk_backward(graph, D, F):
    """dQ, dK, dV of the attention from queries and keys (one head, fp32)
    against the oracle's composition (SDDMM scores, the scores-given
    backward, dQ = A_ds K, dK = A_ds^T Q), with error magnitudes carried
    through the same products."""
    csr = _graphs_for_backward()[graph]
    rng = np.random.default_rng(690 + D)
    Q = rng.standard_normal((csr.n_rows, D)).astype(np.float32)
    K = rng.standard_normal((csr.n_cols, D)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    scale = 0.3
    rp, ci = pattern_dev(csr)
    dQ, dK, dV = csa.attention_qk_backward(rp, ci, dev(Q), dev(K), dev(V), dev(dO), scale=scale)
    th = oracle.default_threads()
    s, _ = oracle.sddmm(csr.row_ptr, csr.col_idx, Q, K, threads=th)
    ds, mag_ds = oracle.attention_backward_scores(csr.row_ptr, csr.col_idx, s.astype(np.float32), V, dO, scale,
                                                  threads=th)
    refQ, _ = oracle.spmm(csr.row_ptr, csr.col_idx, ds, K, threads=th)
    magQ, _ = oracle.spmm(csr.row_ptr, csr.col_idx, mag_ds, np.abs(K), threads=th)
    assert_close(dQ.cpu().numpy(), refQ, magQ, TOL_F32, "dQ")
    refK, _ = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, ds, Q, csr.n_cols)
    magK, _ = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, mag_ds, np.abs(Q), csr.n_cols)
    assert_close(dK.cpu().numpy(), refK, magK, TOL_F32, "dK")
    P = oracle.attention(csr.row_ptr, csr.col_idx, s.astype(np.float32), np.zeros((csr.n_cols, 1), np.float32),
                         scale, want_probs=True, threads=th)[2]
    refV, magV = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, P, dO, csr.n_cols)
    assert_close(dV.cpu().numpy(), refV, magV, TOL_F32, "dV")
    with pytest.raises(ValueError):
        csa.attention_qk_backward(rp, ci, dev(Q), dev(K), dev(V), dev(dO[:-1]))
