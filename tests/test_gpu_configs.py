"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (the schedule chosen by the selector,
replayed): every output element compared with the oracle (computed block by
block over the rows on the host's cores) for the power-law, log-normal and
skew workloads, the single-head fp32 attention on the log-normal graph (scores
given, and the SDDMM -> softmax -> SpMM chains from queries and keys) and the
window attention; for the 8-head attention on the 123.7M-entry graph, a
sample of rows that contains every row the selected partition splits, plus
properties that hold at any size.  The SpMM and SDDMM calls also run through
the library's plan (layout and schedule chosen together), the form bench.py
times."""

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import csr_sparse_attention_amd as csa  # noqa: E402
import oracle  # noqa: E402
from synth import configs  # noqa: E402
from gpu_util import TOL_BF16, TOL_F32, assert_close, bf16_dev, compare_all_rows, dev, max_err  # noqa: E402

THREADS = min(16, oracle.default_threads())


@functools.lru_cache(maxsize=None)
def pattern(name):
    return configs.config_pattern(name)


@functools.lru_cache(maxsize=None)
def pattern_dev(name):
    csr = pattern(name)
    return dev(csr.row_ptr), dev(csr.col_idx)


def sample_rows(csr, n_random=400, n_heavy=24, seed=0):
    deg = csr.degrees()
    rng = np.random.default_rng(seed)
    heavy = np.argsort(deg)[::-1][:n_heavy]
    rand = rng.choice(csr.n_rows, size=min(n_random, csr.n_rows), replace=False)
    empty = np.nonzero(deg == 0)[0][:16]
    ends = np.array([0, csr.n_rows - 1])
    return np.unique(np.concatenate([heavy, rand, empty, ends]))


def split_rows(csr, schedule):
    """Rows whose entries a merge-path partition of the schedule's chunk size
    cuts (a chunk boundary falls strictly inside the row): their results are
    combined from pieces by the fix-up pass."""
    if schedule.mapping == csa.MAP_ROWGROUP:
        return np.zeros(0, dtype=np.int64)
    x, y = oracle.merge_path_partition(csr.row_ptr, schedule.chunk_items)
    x, y = x.astype(np.int64), y.astype(np.int64)
    rp = csr.row_ptr.astype(np.int64)
    ok = x < csr.n_rows
    xs, ys = x[ok], y[ok]
    cut = (rp[xs] < ys) & (ys < rp[xs + 1])
    return np.unique(xs[cut])


def oracle_rows(fn, rows, threads=THREADS):
    """Runs fn(r) -> (value, mag) for every row on a thread pool (the C oracle
    releases the GIL)."""
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(fn, [int(r) for r in rows]))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def selected(op, *args, **kw):
    s, _ = csa.select(op, *args, **kw)
    return s


def planned_format(op, name, rp, ci, a, b):
    csr = pattern(name)
    p, _ = csa.make_problem(op, rp, ci, a, b)
    counts, sums, mx = csa.degree_histogram(rp)
    P, T = csa.hybrid_plan(p, counts + sums + [mx])
    assert P > 1, (name, op, b.shape)
    h = csa.hybrid_format(rp, ci, csr.n_cols, P, whole_below=T)
    if op == "spmm":
        a = None if a is None else csa.hybrid_values(h, a)
    s, _ = csa.hybrid_select(h, op, a, b)
    return h, a, s


# ---------------------------------------------------------------------------
# c2: power-law SpMM, F = 32, 64, 128, 602, on the plain pattern and over the
# column-part segment format, every output element
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("F", [32, 64, 128, 602])
def test_c2_spmm_full(F):
    csr = pattern("c2")
    rp, ci = pattern_dev("c2")
    vals = configs.config_dense("c2", "vals", csr)
    X = configs.config_dense("c2", "X", csr, F)
    vd, Xd = dev(vals), dev(X)
    s = selected("spmm", rp, ci, vd, Xd)
    Y = csa.spmm(rp, ci, vd, Xd, schedule=s).cpu().numpy()
    h, hv, sf = planned_format("spmm", "c2", rp, ci, vd, Xd)
    assert (h.parts, h.whole_below) == {32: (8, 32), 64: (16, 64), 128: (32, 128), 602: (128, 512)}[F]
    # the format at full size: a permutation, segments in (part, row) order
    assert torch.equal(torch.sort(h.perm.long())[0], torch.arange(csr.nnz, device="cuda"))
    assert bool((h.seg_ptr[1:] > h.seg_ptr[:-1]).all()) and int(h.seg_ptr[-1]) == csr.nnz
    assert int(h.row_seg_ptr[-1]) == h.n_seg
    Yf = csa.hybrid_spmm(h, hv, Xd, schedule=sf).cpu().numpy()
    # the library's plan, the call bench.py times
    pl = csa.plan("spmm", rp, ci, vd, Xd)
    Yp = csa.plan_spmm(pl, Xd).cpu().numpy()
    worst = [0.0, 0.0, 0.0]

    def block(r0, r1):
        ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, r0, r1, threads=THREADS)
        worst[1] = max(worst[1], max_err(Yf[r0:r1], ref, mag))
        worst[2] = max(worst[2], max_err(Yp[r0:r1], ref, mag))
        return ref, mag

    worst[0] = compare_all_rows(Y, block, csr.row_ptr, F, TOL_F32, f"c2 F={F}")
    assert worst[1] <= TOL_F32, f"c2 format F={F}: max error {worst[1]:.3e}"
    assert worst[2] <= TOL_F32, f"c2 plan F={F}: max error {worst[2]:.3e}"
    print(f"c2 F={F}: plain {s} max err {worst[0]:.2e}; format P={h.parts} {sf} max err {worst[1]:.2e}; "
          f"{pl} max err {worst[2]:.2e} over all {csr.n_rows} rows")
    # mean aggregation of a constant feature returns the constant on every non-empty row
    ones = torch.ones((csr.n_cols, F), device="cuda")
    Y1 = csa.hybrid_spmm(h, hv, ones, schedule=sf)
    live = torch.from_numpy(csr.degrees() > 0).cuda()
    assert torch.max(torch.abs(Y1[live] - 1.0)).item() < 1e-5
    assert bool((Y1[~live] == 0).all())


# ---------------------------------------------------------------------------
# c3: log-normal symmetric graph, SpMM F = 100, 128 and SDDMM K = 128, every
# output element
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("F", [100, 128])
def test_c3_spmm_full(F):
    csr = pattern("c3")
    rp, ci = pattern_dev("c3")
    vals = configs.config_dense("c3", "vals", csr)
    X = configs.config_dense("c3", "X", csr, F)
    vd, Xd = dev(vals), dev(X)
    s = selected("spmm", rp, ci, vd, Xd)
    Y = csa.spmm(rp, ci, vd, Xd, schedule=s).cpu().numpy()
    pl = csa.plan("spmm", rp, ci, vd, Xd)
    Yp = csa.plan_spmm(pl, Xd).cpu().numpy()
    worst = [0.0]

    def block(r0, r1):
        ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, r0, r1, threads=THREADS)
        worst[0] = max(worst[0], max_err(Yp[r0:r1], ref, mag))
        return ref, mag

    e = compare_all_rows(Y, block, csr.row_ptr, F, TOL_F32, f"c3 F={F}")
    assert worst[0] <= TOL_F32, f"c3 plan F={F}: max error {worst[0]:.3e}"
    print(f"c3 F={F}: {s} max err {e:.2e}; {pl} max err {worst[0]:.2e} over all {csr.n_rows} rows")


@pytest.mark.timeout(900)
def test_c3_sddmm_full():
    csr = pattern("c3")
    rp, ci = pattern_dev("c3")
    U = configs.config_dense("c3", "U", csr, 128)
    V = configs.config_dense("c3", "V", csr, 128)
    Ud, Vd = dev(U), dev(V)
    s = selected("sddmm", rp, ci, Ud, Vd)
    out = csa.sddmm(rp, ci, Ud, Vd, schedule=s).cpu().numpy()
    pl = csa.plan("sddmm", rp, ci, Ud, Vd)
    outp = csa.plan_sddmm(pl, Ud, Vd).cpu().numpy()
    worst = [0.0]
    rp64 = csr.row_ptr.astype(np.int64)

    def block(r0, r1):
        ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, r0, r1, threads=THREADS)
        worst[0] = max(worst[0], max_err(outp[rp64[r0]:rp64[r1]], ref, mag))
        return ref, mag

    e = compare_all_rows(out, block, csr.row_ptr, 128, TOL_F32, "c3 sddmm", per_entry=True)
    assert worst[0] <= TOL_F32, f"c3 plan sddmm: max error {worst[0]:.3e}"
    print(f"c3 sddmm: {s} max err {e:.2e}; {pl} max err {worst[0]:.2e} over all {csr.nnz} entries")


@pytest.mark.timeout(900)
def test_c3_bf16_full():
    """bf16 features on the c3 graph (SpMM F = 128, SDDMM K = 128), fp32
    accumulation: every output element against the oracle reading the same
    bf16 values exactly."""
    from synth import to_bf16_bits

    csr = pattern("c3")
    rp, ci = pattern_dev("c3")
    vals = configs.config_dense("c3", "vals", csr)
    Xb = to_bf16_bits(configs.config_dense("c3", "X", csr, 128))
    Xf = oracle.bf16_to_f32(Xb)
    vd, Xd = dev(vals), bf16_dev(Xb)
    s = selected("spmm", rp, ci, vd, Xd)
    Y = csa.spmm(rp, ci, vd, Xd, schedule=s).cpu().numpy()
    e1 = compare_all_rows(Y, lambda r0, r1: oracle.spmm(csr.row_ptr, csr.col_idx, vals, Xf, r0, r1, threads=THREADS),
                          csr.row_ptr, 128, TOL_BF16, "c3 bf16 spmm")
    del Y
    Ub = to_bf16_bits(configs.config_dense("c3", "U", csr, 128))
    Vb = to_bf16_bits(configs.config_dense("c3", "V", csr, 128))
    Uf, Vf = oracle.bf16_to_f32(Ub), oracle.bf16_to_f32(Vb)
    Ud, Vd = bf16_dev(Ub), bf16_dev(Vb)
    sd = selected("sddmm", rp, ci, Ud, Vd)
    out = csa.sddmm(rp, ci, Ud, Vd, schedule=sd).cpu().numpy()
    e2 = compare_all_rows(out, lambda r0, r1: oracle.sddmm(csr.row_ptr, csr.col_idx, Uf, Vf, r0, r1, threads=THREADS),
                          csr.row_ptr, 128, TOL_BF16, "c3 bf16 sddmm", per_entry=True)
    assert max(e1, e2) <= TOL_F32  # exact bf16 inputs: only fp32 accumulation error remains
    print(f"c3 bf16: spmm {s} max err {e1:.2e}; sddmm {sd} max err {e2:.2e} (all rows / entries)")


# ---------------------------------------------------------------------------
# single-head fp32 attention on the c3 graph, every output element: scores
# given (the fused softmax-aggregation), and from queries and keys as the
# fused (SDDMM -> attention) and unfused (SDDMM -> row softmax -> SpMM) chains
# ---------------------------------------------------------------------------

def _c3_qkv():
    csr = pattern("c3")
    return (csr, configs.config_dense("c3", "U", csr, 64), configs.config_dense("c3", "V", csr, 64),
            configs.config_dense("c3", "X", csr, 64))


@pytest.mark.timeout(900)
def test_c3_attention_scores_full():
    csr = pattern("c3")
    rp, ci = pattern_dev("c3")
    sc = configs.config_dense("c3", "scores", csr) * np.float32(8.0)  # t = 0.125 * s ~ N(0, 1)
    V = configs.config_dense("c3", "X", csr, 64)
    sd, Vd = dev(sc), dev(V)
    s = selected("attention", rp, ci, sd, Vd, scale=0.125)
    out = csa.attention(rp, ci, sd, Vd, scale=0.125, schedule=s).cpu().numpy()

    def block(r0, r1):
        ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, 0.125, r0, r1, threads=THREADS)
        return ref, mag

    e = compare_all_rows(out, block, csr.row_ptr, 64, TOL_F32, "c3 attention")
    print(f"c3 attention (scores given): {s} max err {e:.2e} over all {csr.n_rows} rows")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", ["single", True, False])
def test_c3_attention_chain_full(fused):
    """The same attention from Q, K, V (width 64, scale 1/8) three ways: in one
    pass (scores formed in registers, probabilities written too), as SDDMM then
    the fused softmax-aggregation, and as SDDMM, row softmax and SpMM."""
    csr, Q, K, V = _c3_qkv()
    rp, ci = pattern_dev("c3")
    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    probs = None
    if fused == "single":
        sq = selected("attention_qk", rp, ci, Qd, Kd, Vd, scale=0.125)
        P = torch.empty(csr.nnz, device="cuda")
        out = csa.attention_qk(rp, ci, Qd, Kd, Vd, scale=0.125, probs=P, schedule=sq)
        probs = P.cpu().numpy()
        del P
        label = f"one pass {sq}"
        S = None
    else:
        ss = selected("sddmm", rp, ci, Qd, Kd)
        S = csa.sddmm(rp, ci, Qd, Kd, schedule=ss)
    if fused == "single":
        pass
    elif fused:
        sa = selected("attention", rp, ci, S, Vd, scale=0.125)
        out = csa.attention(rp, ci, S, Vd, scale=0.125, schedule=sa)
        label = f"sddmm {ss}, attention {sa}"
    else:
        P = torch.empty_like(S)
        sp = selected("row_softmax", rp, None, S, scale=0.125, out=P)
        csa.row_softmax(rp, S, scale=0.125, out=P, schedule=sp)
        sm = selected("spmm", rp, ci, P, Vd)
        out = csa.spmm(rp, ci, P, Vd, schedule=sm)
        label = f"sddmm {ss}, softmax {sp}, spmm {sm}"
    out = out.cpu().numpy()
    worst_p = [0.0]

    def block(r0, r1):
        ref, mag, pr = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q, K, V, 0.125, r0, r1, threads=THREADS,
                                           want_probs=probs is not None)
        if probs is not None:
            got = probs[csr.row_ptr[r0]:csr.row_ptr[r1]].astype(np.float64)
            live = pr[:, 0] > 0
            assert np.all(got[~live] == 0)
            d = np.abs(got[live] - pr[live, 0]) / pr[live, 0]
            worst_p[0] = max(worst_p[0], float("inf") if np.isnan(d).any() else float(d.max(initial=0.0)))
        return ref[:, 0], mag[:, 0]

    e = compare_all_rows(out, block, csr.row_ptr, 64, TOL_F32, f"c3 chain fused={fused}")
    assert worst_p[0] <= 1e-5, f"probabilities: {worst_p[0]:.2e}"
    print(f"c3 chain fused={fused}: {label} max err {e:.2e}"
          + (f", probabilities {worst_p[0]:.2e}" if probs is not None else "") + f" over all {csr.n_rows} rows")


# ---------------------------------------------------------------------------
# c4: skew stress, full comparison
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("F", [4, 8, 16, 32])
def test_c4_spmm_full(F):
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    vals = configs.config_dense("c4", "vals", csr)
    X = configs.config_dense("c4", "X", csr, F)
    vd, Xd = dev(vals), dev(X)
    s = selected("spmm", rp, ci, vd, Xd)
    Y = csa.spmm(rp, ci, vd, Xd, schedule=s).cpu().numpy()
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    print(f"c4 spmm F={F}: {s} max err {assert_close(Y, ref, mag, TOL_F32, 'c4 spmm'):.2e}")
    pl = csa.plan("spmm", rp, ci, vd, Xd)
    Yp = csa.plan_spmm(pl, Xd).cpu().numpy()
    print(f"c4 plan spmm F={F}: {pl} max err {assert_close(Yp, ref, mag, TOL_F32, 'c4 plan spmm'):.2e}")


@pytest.mark.parametrize("K", [4, 8, 16, 32])
def test_c4_sddmm_full(K):
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    U = configs.config_dense("c4", "U", csr, K)
    V = configs.config_dense("c4", "V", csr, K)
    s = selected("sddmm", rp, ci, dev(U), dev(V))
    out = csa.sddmm(rp, ci, dev(U), dev(V), schedule=s).cpu().numpy()
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, threads=THREADS)
    print(f"c4 sddmm K={K}: {s} max err {assert_close(out, ref, mag, TOL_F32, 'c4 sddmm'):.2e}")
    Ud, Vd = dev(U), dev(V)
    pl = csa.plan("sddmm", rp, ci, Ud, Vd)
    outp = csa.plan_sddmm(pl, Ud, Vd).cpu().numpy()
    print(f"c4 plan sddmm K={K}: {pl} max err {assert_close(outp, ref, mag, TOL_F32, 'c4 plan sddmm'):.2e}")


def test_c4_format_bit_exact():
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    h = csa.hybrid_format(rp, ci, csr.n_cols, 8, whole_below=16)
    want = oracle.hybrid_format(csr.row_ptr, csr.col_idx, csr.n_cols, 8, whole_below=16)
    assert h.n_seg == len(want["seg_row"])
    for k in ("perm", "col_idx", "seg_ptr", "seg_row", "row_seg_ptr", "row_seg"):
        assert np.array_equal(getattr(h, k).cpu().numpy(), want[k]), k


@pytest.mark.parametrize("F", [4, 8, 16, 32])
def test_c4_spmm_format_full(F):
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    vals = configs.config_dense("c4", "vals", csr)
    X = configs.config_dense("c4", "X", csr, F)
    h, hv, s = planned_format("spmm", "c4", rp, ci, dev(vals), dev(X))
    Y = csa.hybrid_spmm(h, hv, dev(X), schedule=s).cpu().numpy()
    ref, mag = oracle.spmm(csr.row_ptr, csr.col_idx, vals, X, threads=THREADS)
    print(f"c4 format spmm F={F}: P={h.parts} {s} max err {assert_close(Y, ref, mag, TOL_F32, 'c4 format'):.2e}")


@pytest.mark.parametrize("K", [4, 8, 16])
def test_c4_sddmm_format_full(K):
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    U = configs.config_dense("c4", "U", csr, K)
    V = configs.config_dense("c4", "V", csr, K)
    h, Ud, s = planned_format("sddmm", "c4", rp, ci, dev(U), dev(V))
    out = csa.hybrid_sddmm(h, Ud, dev(V), schedule=s).cpu().numpy()
    ref, mag = oracle.sddmm(csr.row_ptr, csr.col_idx, U, V, threads=THREADS)
    print(f"c4 format sddmm K={K}: P={h.parts} {s} max err {assert_close(out, ref, mag, TOL_F32, 'c4 fmt'):.2e}")


# ---------------------------------------------------------------------------
# c5: 8-head bf16 attention on the c3 graph and on the window pattern
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["c5b", "c5a"])
def test_c5_mha(name):
    """c5b (16,384 rows): every output element.  c5a (2,449,029 rows): the
    heaviest rows, a seeded random sample, empty rows, both ends and every
    row the selected partition splits between chunks."""
    csr = pattern(name)
    rp, ci = pattern_dev(name)
    Q = configs.config_dense(name, "Q", csr)
    K = configs.config_dense(name, "K", csr)
    V = configs.config_dense(name, "Vh", csr)
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)
    s = selected("mha", rp, ci, Qd, Kd, Vd, scale=0.125)
    out = csa.mha_attention(rp, ci, Qd, Kd, Vd, scale=0.125, schedule=s)
    if name == "c5b":
        got = out.cpu().numpy()

        def block(r0, r1):
            ref, mag, _ = oracle.mha(csr.row_ptr, csr.col_idx, Q, K, V, 0.125, r0, r1, threads=THREADS)
            return ref, mag

        e = compare_all_rows(got, block, csr.row_ptr, 8 * 64 * 2, TOL_BF16, name)
        where = f"all {csr.n_rows} rows"
    else:
        split = split_rows(csr, s)
        rows = np.unique(np.concatenate([sample_rows(csr, n_random=200, seed=5), split]))
        got = out[torch.from_numpy(rows).cuda()].cpu().numpy()
        ref, mag = oracle_rows(lambda r: oracle.mha(csr.row_ptr, csr.col_idx, Q, K, V, 0.125, r, r + 1)[:2], rows)
        e = assert_close(got, ref, mag, TOL_BF16, name)
        where = f"{len(rows)} rows ({len(split)} split by the partition)"
    assert e < 1e-4  # fp32 accumulation: far inside the bf16 bound
    print(f"{name}: {s} max err {e:.2e} over {where}")


def test_c1_attention_selected():
    c = configs.make_config("c1")
    csr = c["csr"]
    rp, ci = dev(csr.row_ptr), dev(csr.col_idx)
    sd, Vd = dev(c["scores"]), dev(c["V"])
    s = selected("attention", rp, ci, sd, Vd)
    out = csa.attention(rp, ci, sd, Vd, schedule=s).cpu().numpy()
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, c["scores"], c["V"])
    print(f"c1: {s} max err {assert_close(out, ref, mag, TOL_F32, 'c1'):.2e}")


# ---------------------------------------------------------------------------
# row softmax (the unfused pipeline's middle stage) on the c3 and c4 patterns
# ---------------------------------------------------------------------------

def _softmax_case(name, seed):
    csr = pattern(name)
    rp, _ = pattern_dev(name)
    sc = (3 * np.random.default_rng(seed).standard_normal(csr.nnz)).astype(np.float32)
    sd = dev(sc)
    s = selected("row_softmax", rp, None, sd, scale=0.125)
    out = csa.row_softmax(rp, sd, scale=0.125, schedule=s).cpu().numpy()
    return csr, sc, s, out


def _row_sums_ok(csr, out):
    live = csr.degrees() > 0
    sums = np.add.reduceat(out.astype(np.float64), csr.row_ptr[:-1][live])
    return np.max(np.abs(sums - 1))


@pytest.mark.timeout(900)
def test_c3_row_softmax_full():
    csr, sc, s, out = _softmax_case("c3", 31)
    zero = np.zeros((csr.n_cols, 1), np.float32)

    def block(r0, r1):
        p = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, 0.125, r0, r1, threads=THREADS,
                             want_probs=True)[2]
        return p, p

    e = compare_all_rows(out, block, csr.row_ptr, 1, TOL_F32, "c3 row softmax", per_entry=True)
    assert _row_sums_ok(csr, out) < 1e-5
    print(f"c3 row softmax: {s} max err {e:.2e} over all {csr.nnz} entries")


def test_c4_row_softmax_full():
    csr, sc, s, out = _softmax_case("c4", 41)
    zero = np.zeros((csr.n_cols, 1), np.float32)
    ref = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, 0.125, threads=THREADS, want_probs=True)[2]
    err = np.max(np.abs(out.astype(np.float64) - ref) / ref)
    assert err < TOL_F32, err
    assert _row_sums_ok(csr, out) < 1e-5
    print(f"c4 row softmax: {s} max err {err:.2e}")


# ---------------------------------------------------------------------------
# backward operations at full size
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
def test_c3_row_softmax_backward_full():
    csr = pattern("c3")
    rp, _ = pattern_dev("c3")
    rng = np.random.default_rng(33)
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    zero = np.zeros((csr.n_cols, 1), np.float32)
    p = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, 0.125, threads=THREADS,
                         want_probs=True)[2].astype(np.float32)
    g = rng.standard_normal(csr.nnz).astype(np.float32)
    s = selected("row_softmax_backward", rp, None, dev(p), dev(g), scale=0.125)
    out = csa.row_softmax_backward(rp, dev(p), dev(g), scale=0.125, schedule=s).cpu().numpy()
    e = compare_all_rows(out, lambda r0, r1: oracle.softmax_backward(csr.row_ptr, p, g, 0.125, r0, r1,
                                                                   threads=THREADS),
                         csr.row_ptr, 1, TOL_F32, "c3 softmax bwd", per_entry=True)
    print(f"c3 softmax backward: {s} max err {e:.2e} over all {csr.nnz} entries")


def test_c4_attention_backward_full():
    csr = pattern("c4")
    rp, ci = pattern_dev("c4")
    rng = np.random.default_rng(44)
    F = 8
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, F)).astype(np.float32)
    dO = rng.standard_normal((csr.n_rows, F)).astype(np.float32)
    t = csa.transpose(rp, ci, csr.n_cols)
    want = oracle.transpose(csr.row_ptr, csr.col_idx, csr.n_cols)
    for got, exp, name in zip(t, want, ("row_ptr", "col_idx", "perm")):
        assert np.array_equal(got.cpu().numpy(), exp), name
    dS, dV = csa.attention_backward(rp, ci, dev(sc), dev(V), dev(dO), scale=0.125, transposed=t)
    ref, mag = oracle.attention_backward_scores(csr.row_ptr, csr.col_idx, sc, V, dO, 0.125, threads=THREADS)
    e1 = assert_close(dS.cpu().numpy(), ref, mag, TOL_F32, "c4 d scores")
    zero = np.zeros((csr.n_cols, 1), np.float32)
    P = oracle.attention(csr.row_ptr, csr.col_idx, sc, zero, 0.125, threads=THREADS, want_probs=True)[2]
    ref, mag = oracle.spmm_transpose(csr.row_ptr, csr.col_idx, P, dO, csr.n_cols)
    e2 = assert_close(dV.cpu().numpy(), ref, mag, TOL_F32, "c4 dV")
    print(f"c4 attention backward: max err d scores {e1:.2e}, dV {e2:.2e}")
