"""CPU oracle (test infrastructure only).

Plain float64 reference implementations of what the GPU library computes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the library under
``csr_sparse_attention_amd`` never does and shares no code with it.

The arithmetic lives in ``oracle.c`` (built with plain gcc, no fast-math) and,
for the integer bookkeeping of the schedule path, in ``structure.py``.  Each
function here only marshals arguments and splits the row range over threads;
per-row results do not depend on the number of threads.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .structure import (  # noqa: F401
    hybrid_format,
    hybrid_format_loops,
    transpose,
    degree_histogram,
    merge_path_partition,
    merge_path_bruteforce,
    fnv1a64,
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _declare(lib):
    P, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
    lib.oracle_spmm.argtypes = [P, P, P, P, I, I, I, I, P, P]
    lib.oracle_sddmm.argtypes = [P, P, P, I, P, I, I, I, I, P, P]
    lib.oracle_attention.argtypes = [P, P, P, P, I, I, D, I, I, P, P, P]
    lib.oracle_mha.argtypes = [P, P, P, P, P, I, I, D, I, I, P, P, P]
    lib.oracle_attention_qk.argtypes = [P, P, P, P, P, I, I, D, I, I, P, P, P]
    lib.oracle_softmax_backward.argtypes = [P, P, P, D, I, I, P, P]
    lib.oracle_attention_backward.argtypes = [P, P, P, P, P, I, D, I, I, P, P]
    lib.oracle_spmm_transpose.argtypes = [P, P, P, P, I, I, I, P, P]
    for f in (lib.oracle_spmm, lib.oracle_sddmm, lib.oracle_attention, lib.oracle_mha, lib.oracle_attention_qk,
              lib.oracle_softmax_backward, lib.oracle_attention_backward, lib.oracle_spmm_transpose):
        f.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


class use_library:
    """Context manager that routes the functions of this module through
    another build of oracle.c (the pin tests use it to check that planted
    mistakes are caught)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self.saved = _lib
        _lib = _declare(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _ranges(row_ptr, r0, r1, threads):
    """Split [r0, r1) into at most ``threads`` contiguous ranges of similar nnz."""
    if threads <= 1 or r1 - r0 < 2:
        return [(r0, r1)]
    lo, hi = int(row_ptr[r0]), int(row_ptr[r1])
    cuts = [r0]
    for t in range(1, threads):
        target = lo + (hi - lo) * t // threads
        c = int(np.searchsorted(row_ptr[r0:r1 + 1], target, side="left")) + r0
        cuts.append(min(max(c, cuts[-1]), r1))
    cuts.append(r1)
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def _run(parts, fn):
    if len(parts) == 1:
        fn(*parts[0])
        return
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(lambda ab: fn(*ab), parts))


def spmm(row_ptr, col_idx, vals, X, r0=0, r1=None, threads=1):
    """Rows [r0, r1) of Y = A X and their magnitudes sum |a||x| (float64)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    va, Xc = _c(vals, np.float32), np.asarray(X, dtype=np.float32)
    if Xc.ndim != 2 or Xc.strides[1] != 4:
        Xc = np.ascontiguousarray(Xc)
    F, ldx = Xc.shape[1], Xc.strides[0] // 4
    r1 = len(rp) - 1 if r1 is None else r1
    Y = np.zeros((r1 - r0, F))
    M = np.zeros((r1 - r0, F))

    def fn(a, b):
        lib.oracle_spmm(_ptr(rp), _ptr(ci), _ptr(va), _ptr(Xc), F, ldx, a, b,
                        Y[a - r0:].ctypes.data, M[a - r0:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return Y, M


def sddmm(row_ptr, col_idx, U, V, r0=0, r1=None, threads=1):
    """SDDMM values and magnitudes of the stored entries of rows [r0, r1)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    Uc, Vc = _c(U, np.float32), _c(V, np.float32)
    K = Uc.shape[1]
    assert Vc.shape[1] == K
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    n = int(rp[r1]) - base
    out, mag = np.zeros(n), np.zeros(n)

    def fn(a, b):
        off = int(rp[a]) - base
        lib.oracle_sddmm(_ptr(rp), _ptr(ci), _ptr(Uc), K, _ptr(Vc), K, K, a, b,
                         out[off:].ctypes.data, mag[off:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return out, mag


def attention(row_ptr, col_idx, scores, V, scale=1.0, r0=0, r1=None, threads=1,
              want_probs=False):
    """Rows [r0, r1) of softmax_row(scale * S) V with empty rows -> 0.
    Returns (out, mag, probs-or-None)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    sc, Vc = _c(scores, np.float32), _c(V, np.float32)
    F = Vc.shape[1]
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    out, mag = np.zeros((r1 - r0, F)), np.zeros((r1 - r0, F))
    probs = np.zeros(int(rp[r1]) - base) if want_probs else None

    def fn(a, b):
        lib.oracle_attention(_ptr(rp), _ptr(ci), _ptr(sc), _ptr(Vc), F, F, float(scale), a, b,
                             out[a - r0:].ctypes.data, mag[a - r0:].ctypes.data,
                             None if probs is None else probs[int(rp[a]) - base:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return out, mag, probs


def mha(row_ptr, col_idx, Q, K, V, scale, r0=0, r1=None, threads=1, want_probs=False):
    """Multi-head attention from bf16 bit patterns Q, K, V [n, H, D] (uint16).
    Returns (out [rows, H, D], mag, probs [entries, H] or None)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    Qc, Kc, Vc = _c(Q, np.uint16), _c(K, np.uint16), _c(V, np.uint16)
    H, D = Qc.shape[1], Qc.shape[2]
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    out, mag = np.zeros((r1 - r0, H, D)), np.zeros((r1 - r0, H, D))
    probs = np.zeros((int(rp[r1]) - base, H)) if want_probs else None

    def fn(a, b):
        lib.oracle_mha(_ptr(rp), _ptr(ci), _ptr(Qc), _ptr(Kc), _ptr(Vc), H, D, float(scale), a, b,
                       out[a - r0:].ctypes.data, mag[a - r0:].ctypes.data,
                       None if probs is None else probs[int(rp[a]) - base:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return out, mag, probs




def attention_qk(row_ptr, col_idx, Q, K, V, scale, r0=0, r1=None, threads=1, want_probs=False):
    """Attention from fp32 queries and keys: Q [n_rows, H, D] (or [n_rows, D]
    for one head), K, V [n_cols, H, D]; per head, softmax over the row's
    entries of scale * <Q_i, K_j>, then the weighted sum of V rows.
    Returns (out [rows, H, D], mag, probs [entries, H] or None)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    Qc, Kc, Vc = _c(Q, np.float32), _c(K, np.float32), _c(V, np.float32)
    if Qc.ndim == 2:
        Qc, Kc, Vc = Qc[:, None, :], Kc[:, None, :], Vc[:, None, :]
    H, D = Qc.shape[1], Qc.shape[2]
    assert Kc.shape[1:] == (H, D) and Vc.shape[1:] == (H, D)
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    out, mag = np.zeros((r1 - r0, H, D)), np.zeros((r1 - r0, H, D))
    probs = np.zeros((int(rp[r1]) - base, H)) if want_probs else None

    def fn(a, b):
        lib.oracle_attention_qk(_ptr(rp), _ptr(ci), _ptr(Qc), _ptr(Kc), _ptr(Vc), H, D, float(scale), a, b,
                                out[a - r0:].ctypes.data, mag[a - r0:].ctypes.data,
                                None if probs is None else probs[int(rp[a]) - base:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return out, mag, probs


def bf16_to_f32(bits):
    """bfloat16 bit patterns (uint16) widened exactly to float32 (the 16 bits
    become the high half of the float's 32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def softmax_backward(row_ptr, probs, grad, scale=1.0, r0=0, r1=None, threads=1):
    """Softmax backward of the entries of rows [r0, r1) from fp32 probabilities
    and incoming gradient: (values, magnitudes), float64."""
    lib = _load()
    rp = _c(row_ptr, np.int32)
    pc, gc = _c(probs, np.float32), _c(grad, np.float32)
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    n = int(rp[r1]) - base
    out, mag = np.zeros(n), np.zeros(n)

    def fn(a, b):
        off = int(rp[a]) - base
        lib.oracle_softmax_backward(_ptr(rp), _ptr(pc), _ptr(gc), float(scale), a, b,
                                    out[off:].ctypes.data, mag[off:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return out, mag


def attention_backward_scores(row_ptr, col_idx, scores, V, d_out, scale=1.0, r0=0, r1=None, threads=1):
    """Gradient of softmax_row(scale * S) V with respect to the scores for the
    incoming gradient d_out [n_rows, F], entries of rows [r0, r1)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    sc, Vc, dc = _c(scores, np.float32), _c(V, np.float32), _c(d_out, np.float32)
    F = Vc.shape[1]
    assert dc.shape[1] == F
    r1 = len(rp) - 1 if r1 is None else r1
    base = int(rp[r0])
    n = int(rp[r1]) - base
    ds, mag = np.zeros(n), np.zeros(n)

    def fn(a, b):
        off = int(rp[a]) - base
        lib.oracle_attention_backward(_ptr(rp), _ptr(ci), _ptr(sc), _ptr(Vc), _ptr(dc), F, float(scale), a, b,
                                      ds[off:].ctypes.data, mag[off:].ctypes.data)

    _run(_ranges(rp, r0, r1, threads), fn)
    return ds, mag


def spmm_transpose(row_ptr, col_idx, vals, dY, n_cols):
    """A^T dY over the whole matrix (float64 values a_e, None = 1): (dX, mag),
    single-threaded (the columns gather from every row)."""
    lib = _load()
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    va = None if vals is None else np.ascontiguousarray(vals, dtype=np.float64)
    yc = _c(dY, np.float32)
    F = yc.shape[1]
    dX, mag = np.zeros((n_cols, F)), np.zeros((n_cols, F))
    lib.oracle_spmm_transpose(_ptr(rp), _ptr(ci), _ptr(va), _ptr(yc), len(rp) - 1, n_cols, F,
                              dX.ctypes.data, mag.ctypes.data)
    return dX, mag
