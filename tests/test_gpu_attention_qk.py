"""Attention from queries and keys in one pass (csr_attention with no edge
scores: SDDMM -> row-softmax -> SpMM with each score formed in registers and
folded into an online softmax), and the probabilities output of every
attention call, against the oracle: fp32 and bf16, one and several heads,
every schedule the selector may pick on the skew graph (a row of 80,000
entries that every merge-path schedule splits), strided operands."""

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
from test_gpu_parity import pattern_dev, sched_id, schedules, skew_graph  # noqa: E402

THREADS = oracle.default_threads()
TOL_P = 1e-5  # probabilities: relative to the oracle's value


@pytest.fixture(scope="module")
def skew():
    return skew_graph(1)


def probs_close(got, ref, what, rows=None):
    """Relative error of the probabilities; ``rows`` (a bool mask over the
    entries) limits the check to entries whose row's accumulation chain the
    schedule keeps within 4,096 terms (the library's own rule: it offers row
    groups only when no row is longer; a forced row-group schedule on the
    80,000-entry row sums that many fp32 terms in one chain, whose rounding
    alone reaches about 1e-5)."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    live = ref > 0
    if rows is not None:
        live &= rows.reshape(rows.shape + (1,) * (ref.ndim - 1))
        got, ref = np.where(live, got, 0), np.where(live, ref, 0)
    e = float(np.max(np.abs(got[live] - ref[live]) / ref[live])) if live.any() else 0.0
    assert e <= TOL_P, f"{what}: probability error {e:.2e}"
    assert np.all(got[~live] == 0)
    return e


def short_chain_entries(csr, schedule):
    """Entries whose rows a schedule sums in chains of at most 4,096 terms:
    all of them under the merge path (chunks of at most 1,024 items), those of
    rows of at most 4,096 entries under row groups."""
    if schedule is None or schedule.mapping != csa.MAP_ROWGROUP:
        return None
    return np.repeat(csr.degrees() <= 4096, csr.degrees())


def row_sums_ok(csr, p):
    live = csr.degrees() > 0
    sums = np.add.reduceat(np.asarray(p, dtype=np.float64), csr.row_ptr[:-1][live], axis=0)
    return float(np.max(np.abs(sums - 1)))


@pytest.mark.parametrize("D", [1, 4, 16, 64, 100, 256])
def test_attention_qk_every_schedule(skew, D):
    csr = skew
    rng = np.random.default_rng(1100 + D)
    Q = rng.standard_normal((csr.n_rows, D)).astype(np.float32)
    K = rng.standard_normal((csr.n_cols, D)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, D)).astype(np.float32)
    scale = 1.0 / np.sqrt(D)
    ref, mag, pref = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q, K, V, scale, threads=THREADS, want_probs=True)
    ref, mag, pref = ref[:, 0], mag[:, 0], pref[:, 0]
    rp, ci = pattern_dev(csr)
    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    p, _ = csa.make_problem("attention_qk", rp, ci, Qd, Kd, Vd, scale=scale)
    assert p.op == csa._ffi.OP_ATTENTION_QK
    worst = 0.0
    for s in schedules(p):
        P = torch.full((csr.nnz,), float("nan"), device="cuda")
        out = csa.attention_qk(rp, ci, Qd, Kd, Vd, scale=scale, probs=P, schedule=s)
        worst = max(worst, assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s)))
        probs_close(P.cpu().numpy(), pref, sched_id(s), short_chain_entries(csr, s))
    out = csa.attention_qk(rp, ci, Qd, Kd, Vd, scale=scale)  # automatic selection, no probabilities
    assert_close(out.cpu().numpy(), ref, mag, TOL_F32, "auto")
    print(f"attention_qk D={D}: {len(schedules(p))} schedules, max err {worst:.2e}")


@pytest.mark.parametrize("H,D", [(3, 16), (2, 6), (4, 32)])
def test_attention_qk_heads_fp32_strided(skew, H, D):
    """Several fp32 heads (one problem per head on column views, one schedule
    for all), V and out with row strides beyond heads * head_dim, and
    probabilities [nnz, heads]."""
    csr = skew
    rng = np.random.default_rng(1200 + H * D)
    Q = rng.standard_normal((csr.n_rows, H, D)).astype(np.float32)
    K = rng.standard_normal((csr.n_cols, H, D)).astype(np.float32)
    Vw = rng.standard_normal((csr.n_cols, H * D + 6)).astype(np.float32)  # V rows padded
    V = np.ascontiguousarray(Vw[:, :H * D]).reshape(csr.n_cols, H, D)
    ref, mag, pref = oracle.attention_qk(csr.row_ptr, csr.col_idx, Q, K, V, 0.3, threads=THREADS, want_probs=True)
    rp, ci = pattern_dev(csr)
    Vd = dev(Vw)[:, :H * D].view(csr.n_cols, H, D)
    obuf = torch.full((csr.n_rows, H * D + 2), float("nan"), device="cuda")
    out = obuf[:, :H * D].view(csr.n_rows, H, D)
    P = torch.empty((csr.nnz, H), device="cuda")
    csa.attention_qk(rp, ci, dev(Q), dev(K), Vd, scale=0.3, out=out, probs=P)
    assert_close(out.cpu().numpy(), ref, mag, TOL_F32, f"H={H} D={D}")
    probs_close(P.cpu().numpy(), pref, f"H={H} D={D}")
    assert torch.isnan(obuf[:, H * D:]).all()  # nothing written past the heads
    assert row_sums_ok(csr, P.cpu().numpy()) < 1e-5


@pytest.mark.parametrize("H,D", [(8, 64), (2, 6), (1, 1024), (2, 8)])
def test_attention_qk_bf16(skew, H, D):
    """bf16 queries, keys and values: the multi-head kernel where its shape
    rules hold (8 x 64, 2 x 8), the one-pass lane-group kernel otherwise."""
    csr = skew
    rng = np.random.default_rng(1300 + H * D)
    Qb = to_bf16_bits(rng.standard_normal((csr.n_rows, H, D)).astype(np.float32))
    Kb = to_bf16_bits(rng.standard_normal((csr.n_cols, H, D)).astype(np.float32))
    Vb = to_bf16_bits(rng.standard_normal((csr.n_cols, H, D)).astype(np.float32))
    scale = 1.0 / np.sqrt(D)
    Qf, Kf, Vf = (oracle.bf16_to_f32(b) for b in (Qb, Kb, Vb))
    ref, mag, pref = oracle.attention_qk(csr.row_ptr, csr.col_idx, Qf, Kf, Vf, scale, threads=THREADS,
                                         want_probs=True)
    rp, ci = pattern_dev(csr)
    Qd, Kd, Vd = bf16_dev(Qb), bf16_dev(Kb), bf16_dev(Vb)
    p, _ = csa.make_problem("attention_qk", rp, ci, Qd, Kd, Vd, scale=scale)
    want_mha = D & (D - 1) == 0 and 8 <= D <= 512 and H * D <= 512
    assert p.op == (csa._ffi.OP_MHA if want_mha else csa._ffi.OP_ATTENTION_QK)
    for s in schedules(p, thorough=False) if p.op == csa._ffi.OP_ATTENTION_QK else [None]:
        P = torch.empty((csr.nnz, H), device="cuda")
        out = csa.attention_qk(rp, ci, Qd, Kd, Vd, scale=scale, probs=P, schedule=s)
        e = assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, f"bf16 H={H} D={D}")
        assert e <= 1e-4
        probs_close(P.cpu().numpy(), pref, f"bf16 H={H} D={D}", short_chain_entries(csr, s))


@pytest.mark.parametrize("F", [8, 64, 602])
def test_attention_bf16_values_every_schedule(skew, F):
    """Given fp32 scores with bf16 node values."""
    csr = skew
    rng = np.random.default_rng(900 + F)
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    Vb = to_bf16_bits(rng.standard_normal((csr.n_cols, F)).astype(np.float32))
    ref, mag, _ = oracle.attention(csr.row_ptr, csr.col_idx, sc, oracle.bf16_to_f32(Vb), 0.5, threads=THREADS)
    rp, ci = pattern_dev(csr)
    sd, Vd = dev(sc), bf16_dev(Vb)
    p, _ = csa.make_problem("attention", rp, ci, sd, Vd, scale=0.5)
    assert p.dtype == csa._ffi.DTYPE_BF16
    for s in schedules(p):
        out = csa.attention(rp, ci, sd, Vd, scale=0.5, schedule=s)
        e = assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, sched_id(s))
        assert e <= TOL_F32


@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_attention_probs_every_schedule(skew, scale):
    """Given scores: the probabilities of complete rows come from the main
    kernel, those of rows split between chunks from the fix-up."""
    csr = skew
    rng = np.random.default_rng(1400)
    sc = (3 * rng.standard_normal(csr.nnz)).astype(np.float32)
    V = rng.standard_normal((csr.n_cols, 16)).astype(np.float32)
    ref, mag, pref = oracle.attention(csr.row_ptr, csr.col_idx, sc, V, scale, threads=THREADS, want_probs=True)
    rp, ci = pattern_dev(csr)
    sd, Vd = dev(sc), dev(V)
    p, _ = csa.make_problem("attention", rp, ci, sd, Vd, scale=scale)
    for s in schedules(p):
        P = torch.full((csr.nnz,), float("nan"), device="cuda")
        out = csa.attention(rp, ci, sd, Vd, scale=scale, probs=P, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_F32, sched_id(s))
        probs_close(P.cpu().numpy(), pref, sched_id(s), short_chain_entries(csr, s))
        assert row_sums_ok(csr, P.cpu().numpy()) < (1e-5 if s.mapping != csa.MAP_ROWGROUP else 1e-4)


def test_mha_probs_every_mapping(skew):
    csr = skew
    rng = np.random.default_rng(1500)
    H, D = 4, 32
    Qb, Kb, Vb = (to_bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32))
                  for n in (csr.n_rows, csr.n_cols, csr.n_cols))
    ref, mag, pref = oracle.mha(csr.row_ptr, csr.col_idx, Qb, Kb, Vb, 0.2, threads=THREADS, want_probs=True)
    rp, ci = pattern_dev(csr)
    Qd, Kd, Vd = bf16_dev(Qb), bf16_dev(Kb), bf16_dev(Vb)
    p, _ = csa.make_problem("mha", rp, ci, Qd, Kd, Vd, scale=0.2)
    base = csa.default_schedule(p)
    for mapping, chunk in ((csa.MAP_ROWGROUP, 0), (csa.MAP_MERGEPATH, 256), (csa.MAP_MERGEPATH, 1024)):
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        s.mapping, s.chunk_items = mapping, chunk
        P = torch.full((csr.nnz, H), float("nan"), device="cuda")
        out = csa.mha_attention(rp, ci, Qd, Kd, Vd, scale=0.2, probs=P, schedule=s)
        assert_close(out.cpu().numpy(), ref, mag, TOL_BF16, f"mha map {mapping} chunk {chunk}")
        probs_close(P.cpu().numpy(), pref, f"mha map {mapping} chunk {chunk}", short_chain_entries(csr, s))


def test_probs_identity_and_empty_rows():
    """Identity pattern: every probability is exactly 1 and out = V exactly;
    empty rows: zero output, nothing to write."""
    n, D = 500, 16
    rng = np.random.default_rng(1600)
    eye = graphs.CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32))
    rp, ci = pattern_dev(eye)
    Q, K, V = (dev(rng.standard_normal((n, D)).astype(np.float32)) for _ in range(3))
    P = torch.empty(n, device="cuda")
    out = csa.attention_qk(rp, ci, Q, K, V, probs=P)
    assert torch.equal(out, V) and bool((P == 1).all())
    deg = np.where(rng.random(n) < 0.5, 0, rng.integers(1, 6, n))
    csr = graphs.csr_from_degrees(deg, n, rng)
    rp, ci = pattern_dev(csr)
    out = torch.full((n, D), float("nan"), device="cuda")
    csa.attention_qk(rp, ci, Q, K, V, out=out, probs=torch.empty(csr.nnz, device="cuda"))
    empty = torch.from_numpy(deg == 0).cuda()
    assert bool((out[empty] == 0).all()) and not bool(torch.signbit(out[empty]).any())


def test_attention_errors():
    n = 64
    rng = np.random.default_rng(1700)
    csr = graphs.csr_from_degrees(rng.integers(1, 5, n), n, rng)
    rp, ci = pattern_dev(csr)
    Q = dev(rng.standard_normal((n, 2, 8)).astype(np.float32))
    with pytest.raises(ValueError):
        csa.attention_qk(rp, ci, Q, Q, Q, probs=torch.empty(csr.nnz, device="cuda"))  # probs needs [nnz, 2]
    with pytest.raises(TypeError):
        csa.attention_qk(rp, ci, Q, Q.to(torch.bfloat16), Q)
    lib = csa.load_library()
    ctx = csa.default_context()
    out = torch.empty((n, 16), device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    sc = dev(np.zeros((2, csr.nnz), np.float32))  # given scores of 2 heads, head-major
    # several heads of given scores: a leading dimension of V below heads * head_dim is a shape error
    assert lib.csr_attention(ctx.handle, n, n, csr.nnz, rp.data_ptr(), ci.data_ptr(), sc.data_ptr(), None, None,
                             Q.data_ptr(), 0, 2, 8, 8, 1.0, out.data_ptr(), 16, None, None, ws.data_ptr(),
                             ws.numel(), st) == -2
    # no queries
    assert lib.csr_attention(ctx.handle, n, n, csr.nnz, rp.data_ptr(), ci.data_ptr(), None, None, Q.data_ptr(),
                             Q.data_ptr(), 0, 2, 8, 16, 1.0, out.data_ptr(), 16, None, None, ws.data_ptr(),
                             ws.numel(), st) == -1
    torch.cuda.synchronize()
