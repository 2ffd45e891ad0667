"""The C ABI on a machine without a GPU: the library loads and exports every
declared symbol, and its host-side logic (problem and schedule checks, lane
layouts, workspace sizes, signature, schedule cache log) behaves as the
header documents."""

import ctypes
import os
import re
import struct

import numpy as np
import pytest

import csr_sparse_attention_amd as csa
import oracle

_ffi = csa._ffi
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    src = open(os.path.join(ROOT, "include", "csrsa.h")).read()
    return set(re.findall(r"^(?:int|const char\*)\s+(csr_\w+)\(", src, re.M))


def test_library_exports_every_declared_symbol():
    lib = csa.load_library()
    declared = header_symbols()
    assert declared == set(_ffi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = csa.load_library()
    for code in range(0, -13, -1):
        s = lib.csr_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.csr_status_string(-99).decode() == "unknown status"


def problem(op, n_rows=1000, n_cols=1000, nnz=5000, width=64, heads=0, head_dim=0, ld=None, ptr=0x1000):
    p = _ffi.CsrProblem()
    p.op = op
    p.dtype = _ffi.DTYPE_BF16 if op == _ffi.OP_MHA else _ffi.DTYPE_F32
    p.n_rows, p.n_cols, p.nnz, p.width = n_rows, n_cols, nnz, width
    p.heads, p.head_dim = heads, head_dim
    ld = width if ld is None else ld
    p.ld_a = p.ld_b = p.ld_out = ld
    p.a = p.b = p.c = p.out = ptr
    p.scale = 1.0
    return p


@pytest.mark.parametrize("F,vec,W,nv", [
    (1, 1, 1, 1), (2, 2, 1, 1), (3, 1, 4, 1), (4, 4, 1, 1), (6, 2, 4, 1), (32, 4, 8, 1), (64, 4, 16, 1),
    (100, 4, 32, 1), (128, 4, 32, 1), (256, 4, 64, 1), (300, 4, 64, 2), (602, 2, 64, 5), (1024, 4, 64, 4),
    (4096, 4, 64, 16),
])
def test_default_layout(F, vec, W, nv):
    s = csa.default_schedule(problem(_ffi.OP_SPMM, width=F))
    assert (s.vec, s.group_lanes, s.passes) == (vec, W, nv)
    assert s.mapping == _ffi.MAP_MERGEPATH and s.version == _ffi.SCHEDULE_VERSION


@pytest.mark.parametrize("ptr", [0x1000, 0x1004, 0x1008])
@pytest.mark.parametrize("op", [_ffi.OP_SPMM, _ffi.OP_SDDMM, _ffi.OP_ATTENTION])
def test_default_schedule_is_valid_at_every_width(op, ptr):
    # the default is also what a caller may pass back explicitly; widths whose
    # lane count falls between supported pass counts (e.g. 601 one float at a
    # time: 10 passes of 64 lanes, rounded up to 12) must still be accepted
    # (a width no layout covers, e.g. an odd width above 1024, has no default)
    lib = csa.load_library()
    n = ctypes.c_size_t()
    covered = 0
    for F in range(1, 4097):
        p = problem(op, width=F, ptr=ptr)
        s = csa.CsrSchedule()
        rc = lib.csr_default_schedule(None, ctypes.byref(p), ctypes.byref(s))
        if rc == -2:  # CSR_ERR_SHAPE
            assert F > 1024
            continue
        assert rc == 0
        covered += 1
        assert lib.csr_workspace_size(None, ctypes.byref(p), ctypes.byref(s), ctypes.byref(n)) == 0, (F, s.vec,
                                                                                                      s.passes)
    # vec 1 covers widths up to 1024, vec 2 even widths up to 2048, vec 4 multiples of 4 up to 4096
    max_vec = {0x1000: 4, 0x1008: 2, 0x1004: 1}[ptr]
    assert covered == sum(1 for F in range(1, 4097) if any(F % v == 0 and F <= 1024 * v for v in (1, 2, 4)
                                                                if v <= max_vec))


def test_alignment_limits_vector_width():
    s = csa.default_schedule(problem(_ffi.OP_SPMM, width=64, ld=66))
    assert s.vec == 2
    s = csa.default_schedule(problem(_ffi.OP_SPMM, width=64, ptr=0x1004))
    assert s.vec == 1


def test_problem_errors():
    lib = csa.load_library()
    n = ctypes.c_size_t()

    def rc(p):
        return lib.csr_workspace_size(None, ctypes.byref(p), None, ctypes.byref(n))

    assert rc(problem(_ffi.OP_SPMM)) == 0
    assert rc(problem(_ffi.OP_SPMM, width=0)) == -2
    assert rc(problem(_ffi.OP_SPMM, width=4097)) == -2
    assert rc(problem(_ffi.OP_SPMM, width=64, ld=32)) == -2
    assert rc(problem(_ffi.OP_SPMM, nnz=-1)) == -2
    assert rc(problem(_ffi.OP_SPMM, nnz=2**31)) == -2
    p = problem(_ffi.OP_SPMM)
    p.dtype = 7  # no such element type
    assert rc(p) == -3
    for op in (_ffi.OP_SPMM, _ffi.OP_SDDMM, _ffi.OP_ATTENTION):
        p = problem(op)
        p.dtype = _ffi.DTYPE_BF16
        assert rc(p) == 0                        # bf16 operands, fp32 accumulation
        p = problem(op, width=63, ld=64)
        p.dtype = _ffi.DTYPE_BF16
        assert rc(p) == -2                       # bf16 needs an even width
        p = problem(op, width=64, ld=65)
        p.dtype = _ffi.DTYPE_BF16
        assert rc(p) == -4                       # and even leading dimensions
        p = problem(op, ptr=0x1002)
        p.dtype = _ffi.DTYPE_BF16
        assert rc(p) == -4                       # and 4-byte aligned rows
    p = problem(_ffi.OP_ROW_SOFTMAX, width=1)
    p.dtype = _ffi.DTYPE_BF16
    assert rc(p) == -3
    assert rc(problem(_ffi.OP_MHA, width=512, heads=8, head_dim=64)) == 0
    assert rc(problem(_ffi.OP_MHA, width=1024, heads=8, head_dim=128)) == -2
    assert rc(problem(_ffi.OP_MHA, width=8 * 48, heads=8, head_dim=48)) == -2
    assert rc(problem(_ffi.OP_MHA, width=512, heads=8, head_dim=64, ptr=0x1008)) == -4
    p = problem(_ffi.OP_ATTENTION)
    p.scale = float("inf")
    assert rc(p) == -2


@pytest.mark.parametrize("F,ld,ptr,vec,W,nv", [
    (128, 128, 0x1000, 8, 16, 1), (602, 602, 0x1000, 2, 64, 5), (100, 100, 0x1000, 4, 32, 1),
    (512, 512, 0x1000, 8, 64, 1), (4096, 4096, 0x1000, 8, 64, 8), (2, 2, 0x1000, 2, 1, 1),
    (64, 64, 0x1008, 4, 16, 1), (64, 64, 0x1004, 2, 32, 1), (6, 6, 0x1000, 2, 4, 1),
])
def test_default_layout_bf16(F, ld, ptr, vec, W, nv):
    """bf16 operands: the widest of 8, 4, 2 values per lane that the width,
    the leading dimensions and the alignment allow (fp32 outputs written with
    the same layout need 4 * min(vec, 4)-byte alignment)."""
    p = problem(_ffi.OP_SPMM, width=F, ld=ld, ptr=ptr)
    p.dtype = _ffi.DTYPE_BF16
    p.out = 0x1000
    s = csa.default_schedule(p)
    assert (s.vec, s.group_lanes, s.passes) == (vec, W, nv)
    # wide lanes are an fp32 schedule
    assert all(not (c.flags & _ffi.SCHED_WIDE) for c in csa.candidates(p, [0] * 66 + [100]))


def test_attention_qk_and_probs_rules():
    """One head of an attention from queries and keys (a = Q, b = K, c = V):
    widths up to 1024, every leading dimension at least the width, the
    widest access all of Q, K, V and out allow; probabilities only on the
    attention ops, 4-byte aligned."""
    lib = csa.load_library()
    n = ctypes.c_size_t()

    def qk(width=64, ld=64, ld_c=None, ptr=0x1000, dtype=_ffi.DTYPE_F32):
        p = problem(_ffi.OP_ATTENTION_QK, width=width, ld=ld, ptr=ptr)
        p.ld_c = ld if ld_c is None else ld_c
        p.dtype = dtype
        return p

    def rc(p):
        return lib.csr_workspace_size(None, ctypes.byref(p), None, ctypes.byref(n))

    assert rc(qk()) == 0
    assert rc(qk(width=1024, ld=1024)) == 0
    assert rc(qk(width=1025, ld=1025)) == -2
    assert rc(qk(ld_c=32)) == -2                 # V's leading dimension below the width
    assert rc(qk(dtype=_ffi.DTYPE_BF16)) == 0
    assert rc(qk(width=63, ld=64, dtype=_ffi.DTYPE_BF16)) == -2
    p = qk()
    p.c = 0x1002
    assert rc(p) == -4                           # V misaligned
    p = qk(ld=66, ld_c=64)
    assert csa.default_schedule(p).vec == 2      # Q and K rows only 8-byte aligned
    s = csa.default_schedule(qk())
    assert (s.vec, s.group_lanes, s.passes) == (4, 16, 1)
    assert all(c.mapping != _ffi.MAP_SEGSCAN and not c.flags for c in csa.candidates(qk(), [0] * 66 + [100]))
    for op, ok in ((_ffi.OP_ATTENTION, 0), (_ffi.OP_ATTENTION_QK, 0), (_ffi.OP_SPMM, -2), (_ffi.OP_SDDMM, -2)):
        p = qk() if op == _ffi.OP_ATTENTION_QK else problem(op)
        p.probs = 0x2000
        assert rc(p) == ok, op
    p = problem(_ffi.OP_ATTENTION)
    p.probs = 0x2002
    assert rc(p) == -4
    p = problem(_ffi.OP_MHA, width=512, heads=8, head_dim=64)
    p.probs, p.probs_stride = 0x2000, 8
    assert rc(p) == -2                           # the multi-head layout is fixed: [nnz, heads]


def test_workspace_layout_sizes():
    # merge path: 1 KiB head, coords, slot rows, (max, sum) pieces, value pieces
    def up(v):
        return (v + 255) // 256 * 256

    for op, ml_per, val in ((_ffi.OP_SPMM, 0, True), (_ffi.OP_ATTENTION, 2, True), (_ffi.OP_SDDMM, 0, False)):
        p = problem(op, n_rows=10_000, nnz=123_457, width=100)
        s = csa.default_schedule(p)
        nc = -(-(10_000 + 123_457) // s.chunk_items)
        want = 1024 + up((nc + 1) * 8) + up(nc * 8) + up(nc * 2 * ml_per * 4) + (up(nc * 2 * 100 * 4) if val else 0)
        assert csa.workspace_size(p, s) == want
        rg = csa.CsrSchedule.from_buffer_copy(bytes(s))
        rg.mapping, rg.chunk_items, rg.long_row = _ffi.MAP_ROWGROUP, 0, 0
        assert csa.workspace_size(p, rg) == 1024
        assert csa.workspace_size(p) >= csa.workspace_size(p, s)


def test_invalid_schedules_rejected():
    lib = csa.load_library()
    p = problem(_ffi.OP_SPMM, width=64)
    n = ctypes.c_size_t()
    base = csa.default_schedule(p)

    def rc(**kw):
        s = csa.CsrSchedule.from_buffer_copy(bytes(base))
        for k, v in kw.items():
            setattr(s, k, v)
        return lib.csr_workspace_size(None, ctypes.byref(p), ctypes.byref(s), ctypes.byref(n))

    assert rc() == 0
    assert rc(version=2) == -7
    assert rc(op=_ffi.OP_SDDMM) == -7
    assert rc(mapping=3) == -7
    assert rc(chunk_items=300) == -7
    assert rc(group_lanes=3) == -7
    assert rc(group_lanes=128) == -7
    assert rc(passes=7) == -7
    assert rc(group_lanes=4, passes=1) == -7   # does not cover F
    assert rc(group_lanes=16, passes=2) == -7  # empty second pass
    assert rc(group_lanes=8, passes=2) == 0
    assert rc(flags=1) == -7
    assert rc(mapping=_ffi.MAP_ROWGROUP) == -7  # row-group takes chunk = long = 0
    assert rc(mapping=_ffi.MAP_ROWGROUP, chunk_items=0, long_row=0) == 0


def test_signature_is_fnv1a_of_documented_fields():
    p = problem(_ffi.OP_SPMM, n_rows=232_965, n_cols=232_965, nnz=114_600_002, width=602, ptr=0x10000)
    hist = np.arange(67, dtype=np.int64) * 1234567
    sig = csa.signature(p, hist)
    fields = [0x43535253, 1, p.op, p.dtype, p.n_rows, p.n_cols, p.nnz, p.width, 0, 0, 2, 0, 0] + hist.tolist()
    want = oracle.fnv1a64(b"".join(struct.pack("<q", v) for v in fields))
    assert sig == want
    hist2 = hist.copy()
    hist2[5] += 1
    assert csa.signature(p, hist2) != sig
    q = problem(_ffi.OP_MHA, width=512, heads=8, head_dim=64, ptr=0x10000)
    fields = [0x43535253, 1, q.op, q.dtype, q.n_rows, q.n_cols, q.nnz, 512, 8, 64, 8, 0, 0] + hist.tolist()
    assert csa.signature(q, hist) == oracle.fnv1a64(b"".join(struct.pack("<q", v) for v in fields))


def test_device_context_needs_gfx950():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = csa.load_library()
    h = ctypes.c_void_p()
    assert lib.csr_context_create(ctypes.byref(h), 0, None, 0) == -11


def _sched(**kw):
    s = csa.CsrSchedule()
    s.version, s.op, s.mapping, s.vec, s.group_lanes, s.passes, s.chunk_items, s.long_row = 1, 1, 2, 4, 16, 1, 512, 64
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def test_cache_log_robustness(tmp_path):
    path = tmp_path / "cache.log"
    good = "csrsa-cache v1 00000000000000ab op=1 map=2 vec=4 w=16 nv=1 chunk=512 long=64 flags=0 us=12.500\n"
    newer = "csrsa-cache v1 00000000000000ab op=1 map=2 vec=4 w=16 nv=1 chunk=1024 long=64 flags=0 us=10.000\n"
    other = "csrsa-cache v1 00000000000000cd op=3 map=1 vec=2 w=8 nv=1 chunk=0 long=0 flags=0 us=1.000\n"
    lines = [
        "# comment\n",
        good,
        "csrsa-cache v2 00000000000000ef op=1 map=2 vec=4 w=16 nv=1 chunk=512 long=64 flags=0 us=1.0\n",  # schema
        "garbage line\n",
        "csrsa-cache v1 zz op=1\n",
        other,
        newer,
        "csrsa-cache v1 0000000000000011 op=9 map=2 vec=4 w=16 nv=1 chunk=512 long=64 flags=0 us=1.0\n",  # bad op
        "csrsa-cache v1 0000000000000012 op=1 map=2 vec=4 w=16 nv=1 chunk=512 long=64 flags=0 us=1.0 extra\n",
        "csrsa-cache v1 0000000000000013 op=1 map=2 vec=4 w=16 nv=1 chu",  # truncated
    ]
    path.write_text("".join(lines))
    ctx = csa.Context(-1, str(path))
    info = ctx.cache_info()
    assert info["entries"] == 2 and info["skipped_lines"] == 6
    s = ctx.cache_lookup(0xAB)
    assert s.chunk_items == 1024  # the last valid line of a signature wins
    s2 = ctx.cache_lookup(0xCD)
    assert (s2.op, s2.mapping, s2.vec, s2.group_lanes) == (3, 1, 2, 8)
    assert ctx.cache_lookup(0x13) is None
    # store appends one line; a fresh context replays it byte for byte
    t = _sched(chunk_items=256)
    ctx.cache_store(0x77, t)
    ctx.close()
    ctx2 = csa.Context(-1, str(path))
    assert bytes(ctx2.cache_lookup(0x77)) == bytes(t)
    assert bytes(ctx2.cache_lookup(0xAB)) == bytes(_sched(chunk_items=1024))
    ctx2.close()


def test_cache_missing_and_unwritable(tmp_path):
    ctx = csa.Context(-1, str(tmp_path / "does-not-exist-yet.log"))
    assert ctx.cache_info()["entries"] == 0
    ctx.cache_store(1, _sched())
    assert (tmp_path / "does-not-exist-yet.log").exists()
    ctx.close()
    bad = tmp_path / "no-such-dir" / "cache.log"
    ctx = csa.Context(-1, str(bad))
    with pytest.raises(csa.CsrError) as ei:
        ctx.cache_store(2, _sched())
    assert ei.value.code == -9
    assert bytes(ctx.cache_lookup(2)) == bytes(_sched())  # kept in memory
    assert ctx.cache_info()["io_errors"] == 1
    with pytest.raises(csa.CsrError):
        ctx.cache_flush()
    (tmp_path / "no-such-dir").mkdir()
    ctx.cache_flush()  # retried and persisted now
    assert "0000000000000002" in bad.read_text()
    ctx.close()


def test_host_only_context_refuses_operations():
    lib = csa.load_library()
    ctx = csa.Context(-1, None)
    assert lib.csr_spmm(ctx.handle, 1, 1, 0, 0x1000, None, None, 0x1000, 0, 4, 4, 0x1000, 4, None, 0x1000, 4096,
                        None) == -11
    ctx.close()


def _hist_of_degrees(deg):
    counts, sums, mx = oracle.degree_histogram(np.concatenate([[0], np.cumsum(deg)]))
    return np.concatenate([counts, sums, [mx]]).astype(np.int64)


def test_hybrid_parts_rule():
    # measured cost model: gathers from a slice (cheapest at <= 4 MiB per part)
    # against the segments' partial rows, with the segment count expected from
    # the degree histogram; the plain path unless 5 % faster
    from synth import configs, graphs

    def parts(op, deg, n_cols, width, hist=True):
        p = problem(op, n_rows=len(deg), n_cols=n_cols, nnz=int(np.sum(deg)), width=width)
        return csa.hybrid_parts(p, _hist_of_degrees(deg) if hist else None)

    S, D = _ffi.OP_SPMM, _ffi.OP_SDDMM
    # the power-law graph's degrees (~490 entries per row on average): up to 128 parts at F = 602
    pl = graphs.powerlaw_degrees(configs.C2_N, configs.C2_GAMMA, configs.C2_KMAX)
    assert [parts(S, pl, configs.C2_N, F) for F in (32, 64, 128, 602)] == [8, 16, 32, 128]
    assert [parts(D, pl, configs.C2_N, K) for K in (8, 16, 32)] == [1, 4, 1]  # K = 8: 7.5 MB, fits as it is
    # log-normal degrees (~50 per row) and a 1 GB operand: the partial rows
    # would cost more than the gathers save
    ln = graphs.lognormal_degrees(configs.C3_N, configs.C3_MU, configs.C3_SIGMA)
    assert [parts(S, ln, configs.C3_N, F) for F in (64, 100, 128)] == [1, 1, 1]
    # the skew workload's lengths: 30 % empty rows
    sk = np.zeros(configs.C4_N, dtype=np.int64)
    sk[:configs.C4_N - configs.C4_EMPTY] = graphs.rank_size_lengths(configs.C4_N - configs.C4_EMPTY, configs.C4_CAP,
                                                                    configs.C4_NNZ)
    assert [parts(S, sk, configs.C4_N, F) for F in (4, 8, 16, 32)] == [4, 8, 16, 32]
    assert [parts(D, sk, configs.C4_N, K) for K in (4, 8, 16, 32)] == [4, 8, 16, 1]
    # small operand (fits without the format), short rows, other ops
    assert parts(S, np.full(100_000, 50), 100_000, 4) == 1
    assert parts(S, np.full(1_000_000, 3), 1_000_000, 32) == 1
    assert csa.hybrid_parts(problem(_ffi.OP_ATTENTION, n_rows=232_965, n_cols=232_965, nnz=114_600_002, width=32),
                            None) == 1
    # the plan's whole-row threshold: the power-law graph's short rows stay whole
    def plan(op, deg, n_cols, width):
        p = problem(op, n_rows=len(deg), n_cols=n_cols, nnz=int(np.sum(deg)), width=width)
        return csa.hybrid_plan(p, _hist_of_degrees(deg))

    assert [plan(S, pl, configs.C2_N, F) for F in (32, 128, 602)] == [(8, 32), (32, 128), (128, 512)]
    assert [plan(S, sk, configs.C4_N, F) for F in (4, 32)] == [(4, 0), (32, 0)]
    assert plan(D, sk, configs.C4_N, 8) == (8, 0)  # SDDMM splits every row
    assert plan(S, ln, configs.C3_N, 100) == (1, 0)
    # without a histogram every row counts at the mean degree (here: long rows, many segments)
    assert parts(S, pl, configs.C2_N, 602, hist=False) == 64  # 128 with the histogram


def test_hybrid_capacity_and_host_only_context():
    lib = csa.load_library()
    n = ctypes.c_int64()
    assert lib.csr_hybrid_capacity(10, 100, 4, ctypes.byref(n)) == 0 and n.value == 40
    assert lib.csr_hybrid_capacity(1000, 100, 32, ctypes.byref(n)) == 0 and n.value == 100
    assert lib.csr_hybrid_capacity(10, 10_000, 256, ctypes.byref(n)) == 0 and n.value == 2560
    assert lib.csr_hybrid_capacity(0, 0, 1, ctypes.byref(n)) == 0 and n.value == 0
    for bad in ((10, 100, 3), (10, 100, 512), (10, 100, 0), (10, 100, 96), (-1, 100, 4), (10, 2**31, 4)):
        assert lib.csr_hybrid_capacity(*bad, ctypes.byref(n)) == -2
    assert lib.csr_hybrid_capacity(10, 100, 4, None) == -1
    ctx = csa.Context(-1, None)
    b = ctypes.c_size_t()
    assert lib.csr_hybrid_build_workspace_size(ctx.handle, 10, 100, 4, ctypes.byref(b)) == -11
    ctx.close()


def test_context_shared_by_threads():
    # calls on one context from several threads (ctypes drops the GIL during
    # the call): failing and succeeding host-side calls interleave, each
    # returns its own status, and the context stays usable
    import threading

    lib = csa.load_library()
    ctx = csa.Context(-1, None)
    good = problem(_ffi.OP_SPMM, width=602)
    bad = problem(_ffi.OP_SPMM, width=0)
    errors = []

    def work(seed):
        n = ctypes.c_size_t()
        s = csa.CsrSchedule()
        P, T = ctypes.c_int32(), ctypes.c_int32()
        for i in range(2000):
            if (i + seed) % 2:
                rc = lib.csr_workspace_size(ctx.handle, ctypes.byref(bad), None, ctypes.byref(n))
                if rc != -2:
                    errors.append(("bad", rc))
            else:
                if lib.csr_default_schedule(ctx.handle, ctypes.byref(good), ctypes.byref(s)) != 0:
                    errors.append(("default", i))
                if lib.csr_hybrid_plan(ctx.handle, ctypes.byref(good), None, ctypes.byref(P), ctypes.byref(T)) != 0:
                    errors.append(("plan", i))
                if lib.csr_hybrid_build_workspace_size(ctx.handle, 10, 100, 4, ctypes.byref(n)) != -11:
                    errors.append(("host-only", i))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]
    msg = lib.csr_last_error(ctx.handle).decode()
    assert msg  # the message of one of the failed calls
    ctx.close()


@pytest.mark.parametrize("op", [_ffi.OP_SPMM, _ffi.OP_SDDMM, _ffi.OP_ATTENTION])
def test_leading_dimension_bound(op):
    # row strides in bytes fit 32 bits: leading dimensions below 2^30 elements
    lib = csa.load_library()
    n = ctypes.c_size_t()
    ok = problem(op, width=64, ld=(1 << 30) - 64)
    assert lib.csr_workspace_size(None, ctypes.byref(ok), None, ctypes.byref(n)) == 0
    for field in (("ld_a", "ld_b") if op == _ffi.OP_SDDMM else ("ld_b", "ld_out")):
        bad = problem(op, width=64)
        setattr(bad, field, 1 << 30)
        assert lib.csr_workspace_size(None, ctypes.byref(bad), None, ctypes.byref(n)) == -2, field


def test_wide_lane_schedules():
    # 16-byte lanes over rows that are only 4-byte aligned: SpMM row groups of
    # 64 lanes, passes = the fewest supported counts covering width / 256
    lib = csa.load_library()
    n = ctypes.c_size_t()

    def wide(F, passes=None, **kw):
        p = problem(kw.pop("op", _ffi.OP_SPMM), width=F)
        s = csa.CsrSchedule.from_buffer_copy(bytes(csa.default_schedule(p)))
        s.mapping, s.vec, s.group_lanes, s.chunk_items, s.long_row = _ffi.MAP_ROWGROUP, 4, 64, 0, 0
        s.passes = passes if passes is not None else min(v for v in (1, 2, 3, 4, 5, 6, 8, 12, 16)
                                                         if v * 256 >= F)
        s.flags = _ffi.SCHED_WIDE
        for k, v in kw.items():
            setattr(s, k, v)
        return lib.csr_workspace_size(None, ctypes.byref(p), ctypes.byref(s), ctypes.byref(n))

    for F in (4, 5, 602, 777, 1023, 2600, 4096):
        assert wide(F) == 0, F
    assert wide(3) == -7                       # narrower than one vector
    assert wide(602, passes=4) == -7           # not the fewest passes
    assert wide(2600, passes=11) == -7         # unsupported pass count
    assert wide(602, group_lanes=32) == -7
    assert wide(602, vec=2) == -7
    assert wide(602, mapping=_ffi.MAP_MERGEPATH, chunk_items=256) == -7
    assert wide(602, flags=3) == -7            # unknown flag bit
    assert wide(602, op=_ffi.OP_ATTENTION) == -7
    # offered where the operands allow only narrower aligned accesses
    hist = (ctypes.c_int64 * 67)()
    hist[66] = 100
    for F, ld, expect in ((602, 602, True), (600, 600, False), (600, 602, True), (32, 34, False)):
        p = problem(_ffi.OP_SPMM, width=F, ld=ld)
        out = (csa.CsrSchedule * 32)()
        cnt = ctypes.c_int32()
        assert lib.csr_candidates(None, ctypes.byref(p), hist, out, 32, ctypes.byref(cnt)) == 0
        got = [out[i] for i in range(cnt.value) if out[i].flags == _ffi.SCHED_WIDE]
        assert bool(got) == expect, (F, ld)
        for s in got:
            assert (s.vec, s.group_lanes, s.mapping) == (4, 64, _ffi.MAP_ROWGROUP)


def test_value_index_rules():
    """A value index (entry e's value is a[a_idx[e]]) serves SpMM only, must
    be 4-byte aligned and changes the input's signature."""
    lib = csa.load_library()
    n = ctypes.c_size_t()
    for op, code in ((_ffi.OP_SPMM, 0), (_ffi.OP_SDDMM, -2), (_ffi.OP_ATTENTION, -2)):
        p = problem(op, width=32)
        p.a_idx = 0x2000
        assert lib.csr_workspace_size(None, ctypes.byref(p), None, ctypes.byref(n)) == code, op
    p = problem(_ffi.OP_SPMM, width=32)
    p.a_idx = 0x2002
    assert lib.csr_workspace_size(None, ctypes.byref(p), None, ctypes.byref(n)) == -4
    hist = [0] * 66 + [10]
    plain = problem(_ffi.OP_SPMM, width=32)
    idx = problem(_ffi.OP_SPMM, width=32)
    idx.a_idx = 0x2000
    assert csa.signature(plain, hist) != csa.signature(idx, hist)


def _dual(width=64, ld=None, ptr=0x1000):
    p = problem(_ffi.OP_SPMM_SDDMM, width=width, ld=ld, ptr=ptr)
    p.ld_c = width if ld is None else ld
    p.out2 = ptr
    return p


def test_spmm_sddmm_problem_rules():
    """The SpMM + SDDMM problem: fp32 only, U's leading dimension checked like
    X's, the per-entry output (and its index) only for this op and 4-byte
    aligned, schedules on the row-group and merge-path mappings only, the
    SpMM's workspace, and an output index that changes the signature."""
    lib = csa.load_library()
    n = ctypes.c_size_t()

    def ws(p, s=None):
        return lib.csr_workspace_size(None, ctypes.byref(p), None if s is None else ctypes.byref(s), ctypes.byref(n))

    p = _dual()
    assert ws(p) == 0
    d = csa.default_schedule(p)
    assert d.mapping == _ffi.MAP_MERGEPATH and (d.vec, d.group_lanes, d.passes) == (4, 16, 1)
    assert ws(p, d) == 0
    dual_bytes = n.value
    sd = csa.CsrSchedule.from_buffer_copy(bytes(d))
    sd.op = _ffi.OP_SPMM
    assert ws(problem(_ffi.OP_SPMM, width=64), sd) == 0 and n.value == dual_bytes  # the SpMM's carry
    hist = [0] * 33 + [0] * 33 + [100]
    cands = csa.candidates(p, hist)
    assert {c.mapping for c in cands} == {_ffi.MAP_ROWGROUP, _ffi.MAP_MERGEPATH}
    assert all(c.flags == 0 for c in cands)
    for c in cands:
        assert ws(p, c) == 0
    seg = csa.CsrSchedule.from_buffer_copy(bytes(d))
    seg.mapping, seg.group_lanes, seg.passes, seg.long_row, seg.chunk_items = _ffi.MAP_SEGSCAN, 1, 16, 0, 512
    assert ws(p, seg) == -7  # CSR_ERR_SCHEDULE
    bf = _dual()
    bf.dtype = _ffi.DTYPE_BF16
    assert ws(bf) == -3
    short_u = _dual()
    short_u.ld_c = 32
    assert ws(short_u) == -2
    for op in (_ffi.OP_SPMM, _ffi.OP_SDDMM, _ffi.OP_ATTENTION):
        q = problem(op, width=32)
        q.out2 = 0x2000
        assert ws(q) == -2, op
    mis = _dual()
    mis.out2_idx = 0x2002
    assert ws(mis) == -4
    h = [0] * 66 + [10]
    plain, idx = _dual(), _dual()
    idx.out2_idx = 0x2000
    assert csa.signature(plain, h) != csa.signature(idx, h)


def test_backward_calls_check_arguments_on_the_host():
    """csr_spmm_sddmm, csr_inverse_permutation and the permutation plans:
    argument errors before any device work, and a host-only context refuses
    the device calls."""
    lib = csa.load_library()
    ctx = csa.Context(-1, None)
    h = ctx.handle
    P = 0x100000
    # (a missing per-entry output is CSR_ERR_NULL on a device context; the GPU tests check it)
    assert lib.csr_spmm_sddmm(h, 4, 4, 8, P, P, P, None, P, 16, 16, P, 16, P, 16, P, None, None, P, 1 << 20,
                              None) == -11
    assert lib.csr_inverse_permutation(h, -1, P, P + 64, None) == -2
    assert lib.csr_inverse_permutation(h, 8, P, P, None) == -2  # perm and inv alias
    assert lib.csr_inverse_permutation(h, 8, P, None, None) == -1
    assert lib.csr_inverse_permutation(h, 8, P, P + 64, None) == -11
    n = ctypes.c_size_t()
    assert lib.csr_permutation_plan_workspace_size(h, 1 << 31, ctypes.byref(n)) == -2
    assert lib.csr_permutation_plan_workspace_size(h, 100, ctypes.byref(n)) == -11
    for w in (7, 31):
        assert lib.csr_permutation_plan(h, 100, P, w, P + 512, P + 1024, P + 2048, 1 << 20, None) == -2
    assert lib.csr_permutation_plan(h, 100, P, 20, P, P + 1024, P + 2048, 1 << 20, None) == -2  # q and q1 alias
    assert lib.csr_permutation_plan(h, 100, P, 20, P + 512, P + 1024, P + 2048, 1 << 20, None) == -11
    assert lib.csr_permute_values(h, 100, P, P + 512, P + 1024, P + 1024, P + 2048, None) == -2  # src and tmp alias
    assert lib.csr_permute_values(h, 100, P, P + 512, P + 1026, P + 1536, P + 2048, None) == -4  # misaligned
    assert lib.csr_permute_values(h, 100, P, P + 512, P + 1024, P + 1536, P + 2048, None) == -11
    ctx.close()
