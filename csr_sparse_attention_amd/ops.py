"""Python binding of the C ABI: argument marshalling only.

Tensors are passed to the library as device pointers together with their
sizes and leading dimensions; torch provides the memory (outputs and the
workspace) and the current HIP stream.  Every computation happens in
libcsrsa.so; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import NamedTuple, Optional

import torch

from . import _ffi
from ._ffi import CsrError, CsrHybrid, CsrPlan, CsrProblem, CsrSchedule

_lock = threading.Lock()
_contexts: dict = {}
_workspaces: dict = {}
_graph_held: list = []  # workspaces a captured graph refers to: never freed


def _lib():
    return _ffi.load()


def _check(rc: int, where: str, ctx=None):
    if rc != _ffi.CSR_OK:
        msg = ""
        if ctx is not None:
            m = _lib().csr_last_error(ctx.handle)
            msg = m.decode() if m else ""
        raise CsrError(rc, where, msg)


class Context:
    """A library context on one device: schedule cache (optionally persisted
    to ``cache_path``) and the pinned buffer of the auto-select path."""

    def __init__(self, device: int = 0, cache_path: Optional[str] = None, flags: int = 0):
        self.device = device
        self.cache_path = cache_path
        h = ctypes.c_void_p()
        path = cache_path.encode() if cache_path else None
        rc = _lib().csr_context_create(ctypes.byref(h), device, path, flags)
        if rc != _ffi.CSR_OK:
            raise CsrError(rc, "csr_context_create")
        self.handle = h

    def close(self):
        if self.handle:
            _lib().csr_context_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover - interpreter shutdown order
        try:
            self.close()
        except Exception:
            pass

    def cache_info(self):
        e, s, io = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(_lib().csr_cache_info(self.handle, ctypes.byref(e), ctypes.byref(s), ctypes.byref(io)),
               "csr_cache_info", self)
        return {"entries": e.value, "skipped_lines": s.value, "io_errors": io.value}

    def cache_lookup(self, signature: int) -> Optional[CsrSchedule]:
        s = CsrSchedule()
        rc = _lib().csr_cache_lookup(self.handle, ctypes.c_uint64(signature), ctypes.byref(s))
        if rc == _ffi.CSR_ERR_NO_CACHE_ENTRY:
            return None
        _check(rc, "csr_cache_lookup", self)
        return s

    def cache_store(self, signature: int, sched: CsrSchedule):
        _check(_lib().csr_cache_store(self.handle, ctypes.c_uint64(signature), ctypes.byref(sched)),
               "csr_cache_store", self)

    def cache_flush(self):
        _check(_lib().csr_cache_flush(self.handle), "csr_cache_flush", self)


def default_context(device: Optional[int] = None) -> Context:
    """The per-device context used when none is given.  Its cache log is the
    file named by the environment variable CSRSA_CACHE (in memory if unset)."""
    if device is None:
        device = torch.cuda.current_device()
    with _lock:
        ctx = _contexts.get(device)
        if ctx is None:
            ctx = Context(device, os.environ.get("CSRSA_CACHE") or None)
            _contexts[device] = ctx
        return ctx


def _workspace(device: torch.device, nbytes: int, given: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A device buffer of at least nbytes, 256-byte aligned: ``given`` (a
    caller-owned uint8 tensor) when passed, else a buffer cached per (device,
    current stream).  Calls on different streams thus never share scratch
    memory.  A cached buffer is allocated on the stream that uses it, so
    replacing it by a larger one is stream-ordered; a buffer that was handed
    out while the stream was being captured into a graph is kept alive for
    the life of the process, since the graph's replays still write to it."""
    if given is not None:
        if given.dtype != torch.uint8 or not given.is_contiguous() or given.device != device:
            raise ValueError("workspace must be a contiguous uint8 tensor on the operands' device")
        off = (-given.data_ptr()) % 256
        if given.numel() < nbytes + off:
            raise ValueError(f"workspace too small: {given.numel()} bytes, need {nbytes + off}")
        return given[off:]
    stream = torch.cuda.current_stream(device)
    key = (device.index, stream.cuda_stream)
    capturing = torch.cuda.is_current_stream_capturing()
    with _lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes + 256:
            grow = 0 if ws is None else 2 * ws.numel()
            ws = torch.empty(max(nbytes + 256, 1 << 20, grow), dtype=torch.uint8, device=device)
            _workspaces[key] = ws
        if capturing and all(t is not ws for t in _graph_held):
            _graph_held.append(ws)
    off = (-ws.data_ptr()) % 256
    return ws[off:]


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


_DTYPES = {torch.float32: _ffi.DTYPE_F32, torch.bfloat16: _ffi.DTYPE_BF16}


def _dtype_code(t: torch.Tensor, name: str) -> int:
    """The csr_dtype of a dense operand (fp32 or bf16)."""
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    return _DTYPES[t.dtype]


def _dense(t: torch.Tensor, name: str, dtype) -> int:
    """Leading dimension of a row-major 2-D operand (inner stride 1); dtype
    is one torch dtype or a tuple of accepted ones."""
    if t.dtype != dtype and not (isinstance(dtype, tuple) and t.dtype in dtype):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit inner stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _pattern(row_ptr: torch.Tensor, col_idx: torch.Tensor):
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
    if row_ptr.numel() < 1:
        raise ValueError("row_ptr must hold n_rows + 1 >= 1 offsets")
    if col_idx.device != row_ptr.device:
        raise ValueError("row_ptr and col_idx must be on the same device")
    return row_ptr.numel() - 1, col_idx.numel()


# Host-side checks that run before any launch: every row-indexed operand and
# every output has the shape, dtype and element count its call implies, so no
# kernel is handed a buffer shorter than what it reads or writes.

def _on(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the pattern on {device}")


def _rows(t, name, n_rows, width=None, dtype=torch.float32):
    """A row-major 2-D operand of exactly n_rows rows (and width columns);
    dtype is one torch dtype or a tuple of accepted ones."""
    if t.dtype != dtype and not (isinstance(dtype, tuple) and t.dtype in dtype):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[0] != n_rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, the call needs {n_rows}")
    if width is not None and t.shape[1] != width:
        raise ValueError(f"{name} has {t.shape[1]} columns, the call needs {width}")


def _entries(t, name, n):
    """A contiguous fp32 array of exactly n per-entry values."""
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous fp32 tensor of {n} values "
                         f"(got {t.dtype}, {t.numel()} values)")


def _out_rows(out, n_rows, width, device):
    if out is None:
        return torch.empty((n_rows, width), dtype=torch.float32, device=device)
    _on(device, out=out)
    _rows(out, "out", n_rows, width)
    return out


def _out_entries(out, n, device):
    if out is None:
        return torch.empty(n, dtype=torch.float32, device=device)
    _on(device, out=out)
    _entries(out, "out", n)
    return out


def _sched_arg(schedule: Optional[CsrSchedule]):
    return None if schedule is None else ctypes.byref(schedule)


# ---------------------------------------------------------------------------
# problems (shared by the calls, select() and workspace_size())
# ---------------------------------------------------------------------------

def _problem(op: int, row_ptr, col_idx, a, b, c, out, *, n_cols, width, ld_a=0, ld_b=0, ld_out=0,
             heads=0, head_dim=0, scale=1.0, dtype=None) -> CsrProblem:
    p = CsrProblem()
    p.op = op
    if dtype is None:
        dtype = _ffi.DTYPE_BF16 if op == _ffi.OP_MHA else _ffi.DTYPE_F32
    p.dtype = dtype
    p.n_rows = row_ptr.numel() - 1
    p.n_cols = n_cols
    p.nnz = col_idx.numel()
    p.width = width
    p.heads, p.head_dim = heads, head_dim
    p.ld_a, p.ld_b, p.ld_out = ld_a, ld_b, ld_out
    p.row_ptr, p.col_idx = _ptr(row_ptr), _ptr(col_idx)
    p.a, p.b, p.c, p.out = _ptr(a), _ptr(b), _ptr(c), _ptr(out)
    p.scale = scale
    return p


def _spmm_problem(row_ptr, col_idx, vals, X, out):
    ldx = _dense(X, "X", (torch.float32, torch.bfloat16))
    ldy = _dense(out, "out", torch.float32)
    return _problem(_ffi.OP_SPMM, row_ptr, col_idx, vals, X, None, out, n_cols=X.shape[0],
                    width=X.shape[1], ld_b=ldx, ld_out=ldy, dtype=_dtype_code(X, "X"))


def _sddmm_problem(row_ptr, col_idx, U, V, out):
    ldu = _dense(U, "U", (torch.float32, torch.bfloat16))
    ldv = _dense(V, "V", (torch.float32, torch.bfloat16))
    if U.shape[1] != V.shape[1]:
        raise ValueError("U and V must have the same width")
    if U.dtype != V.dtype:
        raise TypeError(f"U and V must have one dtype, got {U.dtype} and {V.dtype}")
    return _problem(_ffi.OP_SDDMM, row_ptr, col_idx, U, V, None, out, n_cols=V.shape[0],
                    width=U.shape[1], ld_a=ldu, ld_b=ldv, dtype=_dtype_code(U, "U"))


def _attention_problem(row_ptr, col_idx, edge_scores, node_value, out, scale, probs=None):
    ldv = _dense(node_value, "node_value", (torch.float32, torch.bfloat16))
    ldo = _dense(out, "out", torch.float32)
    p = _problem(_ffi.OP_ATTENTION, row_ptr, col_idx, edge_scores, node_value, None, out,
                 n_cols=node_value.shape[0], width=node_value.shape[1], ld_b=ldv, ld_out=ldo,
                 scale=scale, dtype=_dtype_code(node_value, "node_value"))
    p.probs, p.probs_stride = _ptr(probs), 1
    return p


def _qk_views(row_ptr, col_idx, Q, K, V, out, probs):
    """Heads H and head_dim D of an attention from queries and keys with
    operands Q [n_rows, (H,) D], K and V [n_cols, (H,) D] (one dtype, fp32 or
    bf16; Q and K rows contiguous), out fp32 [n_rows, (H,) D] and probs fp32
    [nnz, (H)] or None; checks every shape and returns (H, D, ldv, ldo)."""
    n_rows, nnz = row_ptr.numel() - 1, col_idx.numel()
    if Q.dim() not in (2, 3) or K.dim() != Q.dim() or V.dim() != Q.dim():
        raise ValueError("Q, K, V must all be [n, D] or all [n, heads, D]")
    H, D = (1, Q.shape[1]) if Q.dim() == 2 else (Q.shape[1], Q.shape[2])
    if Q.shape[0] != n_rows or K.shape[1:] != Q.shape[1:] or V.shape[1:] != Q.shape[1:] or K.shape[0] != V.shape[0]:
        raise ValueError(f"Q must be [n_rows={n_rows}, ...] and K, V [n_cols, ...] with Q's head shape")
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        _dtype_code(t, name)
        if t.dtype != Q.dtype:
            raise TypeError("Q, K and V must have one dtype")
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != D):
            raise ValueError(f"{name} must have contiguous heads")
    for name, t in (("Q", Q), ("K", K)):
        if t.shape[0] > 1 and t.stride(0) != H * D:
            raise ValueError(f"{name} rows must be contiguous")
    ldv = V.stride(0) if V.shape[0] > 1 else H * D
    if out.dtype != torch.float32 or out.shape != Q.shape or out.stride(-1) != 1 or \
            (out.dim() == 3 and out.stride(1) != D):
        raise ValueError(f"out must be fp32 of Q's shape {tuple(Q.shape)}")
    ldo = out.stride(0) if out.shape[0] > 1 else H * D
    if probs is not None:
        want = (nnz,) if Q.dim() == 2 else (nnz, H)
        if probs.dtype != torch.float32 or not probs.is_contiguous() or tuple(probs.shape) != want:
            raise ValueError(f"probs must be a contiguous fp32 tensor {want}")
    return H, D, ldv, ldo


def _qk_problem(row_ptr, col_idx, Q, K, V, out, probs, scale):
    """The problem the library runs for an attention from queries and keys:
    the multi-head kernel's (bf16, head_dim a power of two in [8, 512],
    heads * head_dim <= 512, contiguous and 16-byte aligned operands), else
    the one-head problem of the head whose column views allow the narrowest
    lane accesses (its schedule serves every head)."""
    H, D, ldv, ldo = _qk_views(row_ptr, col_idx, Q, K, V, out, probs)
    dt = _dtype_code(Q, "Q")
    aligned = all(t.data_ptr() % 16 == 0 for t in (Q, K, V, out))
    if dt == _ffi.DTYPE_BF16 and 8 <= D <= 512 and D & (D - 1) == 0 and H * D <= 512 and ldv == H * D \
            and ldo == H * D and aligned:
        p = _problem(_ffi.OP_MHA, row_ptr, col_idx, Q, K, V, out, n_cols=K.shape[0], width=H * D, heads=H,
                     head_dim=D, scale=scale, dtype=dt)
        p.probs = _ptr(probs)
        return p, H, D, ldv, ldo
    es = Q.element_size()
    best = None
    for h in range(H):
        p = _problem(_ffi.OP_ATTENTION_QK, row_ptr, col_idx, None, None, None, None, n_cols=K.shape[0], width=D,
                     ld_a=H * D, ld_b=H * D, ld_out=ldo, scale=scale, dtype=dt)
        p.a, p.b, p.c = Q.data_ptr() + h * D * es, K.data_ptr() + h * D * es, V.data_ptr() + h * D * es
        p.ld_c = ldv
        p.out = out.data_ptr() + h * D * 4
        p.probs = None if probs is None else probs.data_ptr() + h * 4
        p.probs_stride = H
        s = CsrSchedule()
        _check(_lib().csr_default_schedule(None, ctypes.byref(p), ctypes.byref(s)), "csr_default_schedule")
        if best is None or s.vec < best[0]:
            best = (s.vec, p)
    return best[1], H, D, ldv, ldo


def _mha_problem(row_ptr, col_idx, Q, K, V, out, scale):
    for name, t in (("Q", Q), ("K", K), ("V", V)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor [n, heads, head_dim]")
    H, D = Q.shape[1], Q.shape[2]
    if K.shape[1:] != (H, D) or V.shape[1:] != (H, D) or K.shape[0] != V.shape[0]:
        raise ValueError("Q, K, V shapes do not match")
    return _problem(_ffi.OP_MHA, row_ptr, col_idx, Q, K, V, out, n_cols=K.shape[0], width=H * D,
                    heads=H, head_dim=D, scale=scale)


def _softmax_problem(row_ptr, scores, out, scale):
    p = CsrProblem()
    p.op = _ffi.OP_ROW_SOFTMAX
    p.dtype = _ffi.DTYPE_F32
    p.n_rows = row_ptr.numel() - 1
    p.nnz = scores.numel()
    p.width = 1
    p.row_ptr, p.a, p.out = _ptr(row_ptr), _ptr(scores), _ptr(out)
    p.scale = scale
    return p


def _run(problem: CsrProblem, device, schedule, ctx, call, workspace=None):
    ctx = ctx or default_context(device.index)
    lib = _lib()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_workspace_size(ctx.handle, ctypes.byref(problem), _sched_arg(schedule), ctypes.byref(nbytes)),
           "csr_workspace_size", ctx)
    ws = _workspace(device, nbytes.value, workspace)
    rc = call(ctx, ws, nbytes.value, _stream(device))
    _check(rc, "csr call", ctx)


# ---------------------------------------------------------------------------
# public calls
# ---------------------------------------------------------------------------

def spmm(row_ptr, col_idx, vals, X, *, val_idx=None, out=None, schedule: Optional[CsrSchedule] = None,
         ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = A X for the CSR matrix A (row_ptr, col_idx, vals; vals=None means 1).
    X is float32 or bfloat16 (fp32 accumulation); Y is float32.  With
    ``val_idx`` (int32 [nnz], indices in [0, nnz)) entry e's value is
    vals[val_idx[e]] (csr_spmm_perm): with a transposed pattern and its perm,
    A^T X over values kept in A's order."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, vals=vals, X=X, val_idx=val_idx)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [n_cols, F]")
    if vals is not None:
        _entries(vals, "vals", nnz)
    if val_idx is not None:
        if vals is None:
            raise ValueError("val_idx needs vals")
        if val_idx.dtype != torch.int32 or val_idx.dim() != 1 or not val_idx.is_contiguous() \
                or val_idx.numel() != nnz:
            raise ValueError(f"val_idx must be a contiguous 1-D int32 tensor of {nnz} entries")
    out = _out_rows(out, n_rows, X.shape[1], X.device)
    p = _spmm_problem(row_ptr, col_idx, vals, X, out)
    if val_idx is not None:
        p.a_idx = val_idx.data_ptr()

    def call(ctx, ws, nb, st):
        if val_idx is not None:
            return _lib().csr_spmm_perm(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.a_idx,
                                        p.b, p.dtype, p.width, p.ld_b, p.out, p.ld_out, _sched_arg(schedule),
                                        ws.data_ptr(), nb, st)
        return _lib().csr_spmm(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.b, p.dtype,
                               p.width, p.ld_b, p.out, p.ld_out, _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, X.device, schedule, ctx, call, workspace)
    return out


def _index_arg(t, name, nnz):
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.numel() != nnz:
        raise ValueError(f"{name} must be a contiguous 1-D int32 tensor of {nnz} entries")


def _spmm_sddmm_problem(row_ptr, col_idx, vals, X, U, out, z, val_idx, z_idx):
    ldx = _dense(X, "X", torch.float32)
    ldu = _dense(U, "U", torch.float32)
    ldy = _dense(out, "out", torch.float32)
    p = _problem(_ffi.OP_SPMM_SDDMM, row_ptr, col_idx, vals, X, U, out, n_cols=X.shape[0], width=X.shape[1],
                 ld_b=ldx, ld_out=ldy)
    p.ld_c = ldu
    p.a_idx, p.out2, p.out2_idx = _ptr(val_idx), _ptr(z), _ptr(z_idx)
    return p


def spmm_sddmm(row_ptr, col_idx, vals, X, U, *, val_idx=None, z_idx=None, out=None, z=None,
               schedule: Optional[CsrSchedule] = None, ctx: Optional[Context] = None,
               workspace: Optional[torch.Tensor] = None):
    """Y = A X and z_e = <U[row_e], X[col_e]> from one read of each gathered
    row of X (csr_spmm_sddmm; fp32).  vals=None means 1; with ``val_idx``
    entry e's value is vals[val_idx[e]]; with ``z_idx`` (distinct indices in
    [0, nnz)) z_e is written at z[z_idx[e]].  X [n_cols, F], U [n_rows, F];
    returns (Y [n_rows, F], z [nnz])."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, vals=vals, X=X, U=U, val_idx=val_idx, z_idx=z_idx, out=out, z=z)
    if X.dim() != 2 or U.dim() != 2:
        raise ValueError("X and U must be 2-D")
    if U.shape[0] != n_rows or U.shape[1] != X.shape[1]:
        raise ValueError(f"U must be [n_rows={n_rows}, F={X.shape[1]}]")
    if vals is not None:
        _entries(vals, "vals", nnz)
    if val_idx is not None:
        if vals is None:
            raise ValueError("val_idx needs vals")
        _index_arg(val_idx, "val_idx", nnz)
    if z_idx is not None:
        _index_arg(z_idx, "z_idx", nnz)
    out = _out_rows(out, n_rows, X.shape[1], X.device)
    if z is None:
        z = torch.empty(nnz, dtype=torch.float32, device=X.device)
    _entries(z, "z", nnz)
    p = _spmm_sddmm_problem(row_ptr, col_idx, vals, X, U, out, z, val_idx, z_idx)

    def call(ctx, ws, nb, st):
        return _lib().csr_spmm_sddmm(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.a_idx,
                                     p.b, p.width, p.ld_b, p.c, p.ld_c, p.out, p.ld_out, p.out2, p.out2_idx,
                                     _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, X.device, schedule, ctx, call, workspace)
    return out, z


def spmm_noalloc(row_ptr, col_idx, vals, X, *, schedule: CsrSchedule, out=None,
                 ctx: Optional[Context] = None) -> torch.Tensor:
    """spmm without a workspace (csr_spmm_noalloc): the kernels' scratch lives
    in a fixed device array inside the library (CSR_NOALLOC_SCRATCH_BYTES per
    GPU), so the call allocates nothing but ``out`` when it is not given.  A
    schedule is required.  Calls overlapping on one GPU share the array and
    must be ordered by the caller."""
    if schedule is None:
        raise ValueError("spmm_noalloc needs an explicit schedule (select() one beforehand)")
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, vals=vals, X=X)
    if X.dim() != 2:
        raise ValueError("X must be 2-D [n_cols, F]")
    if vals is not None:
        _entries(vals, "vals", nnz)
    out = _out_rows(out, n_rows, X.shape[1], X.device)
    p = _spmm_problem(row_ptr, col_idx, vals, X, out)
    ctx = ctx or default_context(X.device.index)
    _check(_lib().csr_spmm_noalloc(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.b, p.dtype,
                                   p.width, p.ld_b, p.out, p.ld_out, ctypes.byref(schedule), _stream(X.device)),
           "csr_spmm_noalloc", ctx)
    return out


def sddmm(row_ptr, col_idx, U, V, *, out=None, schedule: Optional[CsrSchedule] = None,
          ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[e] = <U[row(e)], V[col_idx[e]]> for every stored entry e (U and V
    both float32 or both bfloat16; fp32 accumulation and output)."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, U=U, V=V)
    _rows(U, "U", n_rows, dtype=(torch.float32, torch.bfloat16))
    if V.dim() != 2:
        raise ValueError("V must be 2-D [n_cols, K]")
    out = _out_entries(out, nnz, U.device)
    p = _sddmm_problem(row_ptr, col_idx, U, V, out)

    def call(ctx, ws, nb, st):
        return _lib().csr_sddmm(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.ld_a,
                                p.b, p.ld_b, p.dtype, p.width, p.out, _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, U.device, schedule, ctx, call, workspace)
    return out


def attention(row_ptr, col_idx, edge_scores, node_value, *, scale: float = 1.0, out=None, probs=None,
              schedule: Optional[CsrSchedule] = None, ctx: Optional[Context] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused CSR attention with given scores: per row, softmax over the row's
    entries of scale * edge_scores, then the weighted sum of node_value rows
    (fp32 or bf16; zero for rows without entries).  Arguments in the order
    row_ptr, col_idx, edge_scores, node_value.  ``probs`` (fp32 [nnz]), when
    given, receives every entry's probability.  Several heads: edge_scores
    [H, nnz] (head-major), node_value [n_cols, H, D] -> out [n_rows, H, D],
    probs [nnz, H]."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, edge_scores=edge_scores, node_value=node_value, probs=probs, out=out)
    if edge_scores.dim() == 2:
        return _attention_heads(row_ptr, col_idx, edge_scores, node_value, n_rows, nnz, scale, out, probs,
                                schedule, ctx, workspace)
    _entries(edge_scores, "edge_scores", nnz)
    if node_value.dim() != 2:
        raise ValueError("node_value must be 2-D [n_cols, F]")
    if probs is not None:
        _entries(probs, "probs", nnz)
    out = _out_rows(out, n_rows, node_value.shape[1], node_value.device)
    p = _attention_problem(row_ptr, col_idx, edge_scores, node_value, out, scale, probs)

    def call(ctx, ws, nb, st):
        return _lib().csr_attention(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, None, None,
                                    p.b, p.dtype, 1, p.width, p.ld_b, ctypes.c_float(scale), p.out, p.ld_out,
                                    _ptr(probs), _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, node_value.device, schedule, ctx, call, workspace)
    return out


def _attention_heads(row_ptr, col_idx, scores, V, n_rows, nnz, scale, out, probs, schedule, ctx, workspace):
    """attention() over several heads of given scores (csr_attention, heads > 1)."""
    H = scores.shape[0]
    if scores.dtype != torch.float32 or scores.shape[1] != nnz or not scores.is_contiguous():
        raise ValueError(f"edge_scores must be contiguous float32 [heads, {nnz}]")
    if V.dim() != 3 or V.shape[1] != H or V.stride(2) != 1 or V.stride(1) != V.shape[2]:
        raise ValueError(f"node_value must be [n_cols, {H}, D] with contiguous heads")
    D = V.shape[2]
    V2 = V.view(V.shape[0], H * D) if V.shape[0] > 0 else V.reshape(0, H * D)
    if out is None:
        out = torch.empty((n_rows, H, D), dtype=torch.float32, device=V.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (n_rows, H, D) or out.stride(2) != 1 \
            or out.stride(1) != D:
        raise ValueError(f"out must be float32 [{n_rows}, {H}, {D}] with contiguous heads")
    out2 = out.view(n_rows, H * D) if n_rows > 0 else out.reshape(0, H * D)
    if probs is not None and (probs.dtype != torch.float32 or tuple(probs.shape) != (nnz, H)
                              or not probs.is_contiguous()):
        raise ValueError(f"probs must be contiguous float32 [{nnz}, {H}]")
    # the problem of head 0 (every head shares its shape, strides and schedule)
    p = _attention_problem(row_ptr, col_idx, scores, V2[:, :D], out2[:, :D], scale, None)
    ldv, ldo = V2.stride(0) if V2.shape[0] > 1 else H * D, out2.stride(0) if n_rows > 1 else H * D

    def call(ctx, ws, nb, st):
        return _lib().csr_attention(ctx.handle, n_rows, V.shape[0], nnz, row_ptr.data_ptr(), col_idx.data_ptr(),
                                    scores.data_ptr(), None, None, V.data_ptr(), p.dtype, H, D, ldv,
                                    ctypes.c_float(scale), out.data_ptr(), ldo, _ptr(probs), _sched_arg(schedule),
                                    ws.data_ptr(), nb, st)

    _run(p, V.device, schedule, ctx, call, workspace)
    return out


def attention_qk(row_ptr, col_idx, Q, K, V, *, scale: Optional[float] = None, out=None, probs=None,
                 schedule: Optional[CsrSchedule] = None, ctx: Optional[Context] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """CSR attention from queries and keys in one pass (SDDMM -> row-softmax ->
    SpMM with the scores formed on the fly): Q [n_rows, D] or [n_rows, H, D],
    K and V [n_cols, (H,) D], all fp32 or all bf16; per head, softmax over the
    row's entries of scale * <Q_i, K_j> (scale defaults to 1/sqrt(D)), then the
    weighted sum of V rows (fp32 accumulation).  Returns fp32 of Q's shape.
    ``probs`` (fp32 [nnz] or [nnz, H]) receives the probabilities."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, Q=Q, K=K, V=V, out=out, probs=probs)
    if scale is None:
        scale = 1.0 / float(Q.shape[-1]) ** 0.5
    if out is None:
        out = torch.empty(tuple(Q.shape), dtype=torch.float32, device=Q.device)
    p, H, D, ldv, ldo = _qk_problem(row_ptr, col_idx, Q, K, V, out, probs, scale)

    def call(ctx, ws, nb, st):
        return _lib().csr_attention(ctx.handle, n_rows, K.shape[0], nnz, row_ptr.data_ptr(), col_idx.data_ptr(),
                                    None, Q.data_ptr(), K.data_ptr(), V.data_ptr(), p.dtype, H, D, ldv,
                                    ctypes.c_float(scale), out.data_ptr(), ldo, _ptr(probs), _sched_arg(schedule),
                                    ws.data_ptr(), nb, st)

    _run(p, Q.device, schedule, ctx, call, workspace)
    return out


def mha_attention(row_ptr, col_idx, Q, K, V, *, scale: Optional[float] = None, out=None, probs=None,
                  schedule: Optional[CsrSchedule] = None, ctx: Optional[Context] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Multi-head fused CSR attention: bf16 Q [n_rows, H, D], K, V [n_cols, H, D];
    per head, softmax over the row's entries of scale * <Q_i, K_j>, times V.
    Returns fp32 [n_rows, H, D].  scale defaults to 1/sqrt(D).  ``probs``
    (fp32 [nnz, H]) receives the probabilities."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    _on(row_ptr.device, Q=Q, K=K, V=V)
    if Q.dim() != 3 or Q.shape[0] != n_rows:
        raise ValueError(f"Q must be [n_rows={n_rows}, heads, head_dim], got {tuple(Q.shape)}")
    H, D = Q.shape[1], Q.shape[2]
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((n_rows, H, D), dtype=torch.float32, device=Q.device)
    _on(row_ptr.device, out=out)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (n_rows, H, D):
        raise ValueError(f"out must be a contiguous fp32 tensor [{n_rows}, {H}, {D}]")
    if probs is not None:
        _on(row_ptr.device, probs=probs)
        if probs.dtype != torch.float32 or not probs.is_contiguous() or tuple(probs.shape) != (nnz, H):
            raise ValueError(f"probs must be a contiguous fp32 tensor [{nnz}, {H}]")
    p = _mha_problem(row_ptr, col_idx, Q, K, V, out, scale)
    p.probs = _ptr(probs)

    def call(ctx, ws, nb, st):
        return _lib().csr_mha_attention(ctx.handle, p.n_rows, p.n_cols, p.nnz, p.row_ptr, p.col_idx, p.a, p.b,
                                        p.c, H, D, ctypes.c_float(scale), p.out, _ptr(probs),
                                        _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, Q.device, schedule, ctx, call, workspace)
    return out


def row_softmax(row_ptr, scores, *, scale: float = 1.0, out=None, schedule: Optional[CsrSchedule] = None,
                ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-row softmax over the stored entries: out[e] = exp(scale * s_e - m_i) /
    sum over row i of exp(scale * s - m_i).  ``out`` may be ``scores`` (in place)."""
    _pattern(row_ptr, row_ptr)
    _on(row_ptr.device, scores=scores)
    if scores.dtype != torch.float32 or scores.dim() != 1 or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous 1-D fp32 tensor")
    out = _out_entries(out, scores.numel(), scores.device)
    p = _softmax_problem(row_ptr, scores, out, scale)

    def call(ctx, ws, nb, st):
        return _lib().csr_row_softmax(ctx.handle, p.n_rows, p.nnz, p.row_ptr, p.a, ctypes.c_float(scale), p.out,
                                      _sched_arg(schedule), ws.data_ptr(), nb, st)

    _run(p, scores.device, schedule, ctx, call, workspace)
    return out


def attention_pipeline(row_ptr, col_idx, Q, K, V, *, scale: float = 1.0, fused=True,
                       ctx: Optional[Context] = None) -> torch.Tensor:
    """Single-head fp32 CSR attention from Q [n_rows, d], K [n_cols, d],
    V [n_cols, F] as the composition of library calls SDDMM -> row-softmax ->
    SpMM.  fused="single" runs the one-pass kernel (``attention_qk``: the
    scores never leave the registers; needs F == d); fused=True runs SDDMM
    then the fused softmax-aggregation (``attention``); fused=False runs the
    three stages separately."""
    if fused == "single":
        return attention_qk(row_ptr, col_idx, Q, K, V, scale=scale, ctx=ctx)
    scores = sddmm(row_ptr, col_idx, Q, K, ctx=ctx)
    if fused:
        return attention(row_ptr, col_idx, scores, V, scale=scale, ctx=ctx)
    probs = row_softmax(row_ptr, scores, scale=scale, out=scores, ctx=ctx)
    return spmm(row_ptr, col_idx, probs, V, ctx=ctx)


# ---------------------------------------------------------------------------
# backward operations
# ---------------------------------------------------------------------------

def _softmax_bwd_problem(row_ptr, probs, grad, out, scale):
    p = _softmax_problem(row_ptr, probs, out, scale)
    p.op = _ffi.OP_SOFTMAX_BWD
    p.b = _ptr(grad)
    return p


def _flat_f32(t, name, n):
    if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name} must be a contiguous 1-D fp32 tensor of {n} values")


def row_softmax_backward(row_ptr, probs, grad, *, scale: float = 1.0, out=None,
                         schedule: Optional[CsrSchedule] = None, ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the row softmax: out[e] = scale * p_e * (g_e - sum over the
    row of p g), for p = row_softmax(s, scale) and g = dL/dp.  ``out`` may be
    ``probs`` or ``grad`` (in place)."""
    _pattern(row_ptr, row_ptr)
    _on(row_ptr.device, probs=probs, grad=grad)
    _flat_f32(probs, "probs", probs.numel())
    _flat_f32(grad, "grad", probs.numel())
    out = _out_entries(out, probs.numel(), probs.device)
    p = _softmax_bwd_problem(row_ptr, probs, grad, out, scale)

    def call(ctx, ws, nb, st):
        return _lib().csr_row_softmax_backward(ctx.handle, p.n_rows, p.nnz, p.row_ptr, p.a, p.b,
                                               ctypes.c_float(scale), p.out, _sched_arg(schedule), ws.data_ptr(),
                                               nb, st)

    _run(p, probs.device, schedule, ctx, call, workspace)
    return out


class PermutationPlan(NamedTuple):
    """dst[e] = src[q[e]] in two passes (csr_permutation_plan): q1 and pos,
    int32 [n] each."""
    q1: torch.Tensor
    pos: torch.Tensor


class Transposed(NamedTuple):
    """The CSR pattern of A^T: row_ptr [n_cols + 1], col_idx [nnz] (rows of A)
    and perm [nnz] (the entry of A behind each entry of A^T); inv [nnz] (the
    position in A^T of each entry of A, perm's inverse) when asked for; with
    plans, to_t moves per-entry values of A into A^T's order and from_t back
    (two-pass permutations of perm and inv)."""
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    perm: torch.Tensor
    inv: Optional[torch.Tensor] = None
    to_t: Optional[PermutationPlan] = None
    from_t: Optional[PermutationPlan] = None


def transpose(row_ptr, col_idx, n_cols: int, *, inverse: bool = False, plans: bool = False,
              ctx: Optional[Context] = None) -> Transposed:
    """CSR of A^T for the pattern (row_ptr, col_idx) with n_cols columns; the
    entries of each column keep their row order (deterministic).  row_ptr is
    checked only on a validating context; without the check, and with col_idx
    in range, a row_ptr that is not monotone still yields rows in
    [0, n_rows) and a permutation of the entries (which rows is unspecified).
    ``inverse``: also the inverse of perm (csr_inverse_permutation);
    ``plans``: also the two-pass permutation plans of perm and its inverse."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    lib = _lib()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_transpose_workspace_size(ctx.handle, n_rows, n_cols, nnz, ctypes.byref(nbytes)),
           "csr_transpose_workspace_size", ctx)
    ws = _workspace(device, nbytes.value)
    t_rp = torch.empty(n_cols + 1, dtype=torch.int32, device=device)
    t_ci = torch.empty(nnz, dtype=torch.int32, device=device)
    perm = torch.empty(nnz, dtype=torch.int32, device=device)
    _check(lib.csr_transpose(ctx.handle, n_rows, n_cols, nnz, row_ptr.data_ptr(), col_idx.data_ptr(),
                             t_rp.data_ptr(), t_ci.data_ptr(), perm.data_ptr(), ws.data_ptr(), nbytes.value,
                             _stream(device)), "csr_transpose", ctx)
    inv = inverse_permutation(perm, ctx=ctx) if (inverse or plans) else None
    if not plans:
        return Transposed(t_rp, t_ci, perm, inv)
    return Transposed(t_rp, t_ci, perm, inv, permutation_plan(perm, ctx=ctx), permutation_plan(inv, ctx=ctx))


def permutation_plan(q, *, window_log2: int = 22, ctx: Optional[Context] = None) -> PermutationPlan:
    """The two-pass plan of dst[e] = src[q[e]] for a permutation q of [0, n)
    (int32 on the GPU): outputs grouped by the window of 2^window_log2 source
    values they read (csr_permutation_plan).  The default, 16 MiB windows of
    fp32 values, was the fastest on a 123.7M-entry transpose (1.26 ms per
    permutation against 1.46 with 1 MiB and 1.91 with 64 MiB windows, and
    2.26 ms for the direct gather)."""
    if q.dtype != torch.int32 or q.dim() != 1 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous 1-D int32 GPU tensor")
    n = q.numel()
    ctx = ctx or default_context(q.device.index)
    lib = _lib()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_permutation_plan_workspace_size(ctx.handle, n, ctypes.byref(nbytes)),
           "csr_permutation_plan_workspace_size", ctx)
    ws = _workspace(q.device, nbytes.value)
    q1, pos = torch.empty_like(q), torch.empty_like(q)
    _check(lib.csr_permutation_plan(ctx.handle, n, q.data_ptr(), window_log2, q1.data_ptr(), pos.data_ptr(),
                                    ws.data_ptr(), nbytes.value, _stream(q.device)), "csr_permutation_plan", ctx)
    return PermutationPlan(q1, pos)


def permute_values(plan: PermutationPlan, src, *, out=None, tmp=None, ctx: Optional[Context] = None) -> torch.Tensor:
    """out[e] = src[q[e]] through a permutation plan (csr_permute_values; fp32)."""
    n = plan.q1.numel()
    _on(plan.q1.device, src=src, out=out, tmp=tmp, pos=plan.pos)
    _entries(src, "src", n)
    _index_arg(plan.pos, "pos", n)
    out = _out_entries(out, n, src.device)
    tmp = _out_entries(tmp, n, src.device)
    ctx = ctx or default_context(src.device.index)
    _check(_lib().csr_permute_values(ctx.handle, n, plan.q1.data_ptr(), plan.pos.data_ptr(), src.data_ptr(),
                                     tmp.data_ptr(), out.data_ptr(), _stream(src.device)), "csr_permute_values", ctx)
    return out


def inverse_permutation(perm, *, out=None, ctx: Optional[Context] = None) -> torch.Tensor:
    """inv[perm[k]] = k for a permutation perm of [0, n) (int32 on the GPU)."""
    if perm.dtype != torch.int32 or perm.dim() != 1 or not perm.is_contiguous() or not perm.is_cuda:
        raise ValueError("perm must be a contiguous 1-D int32 GPU tensor")
    if out is None:
        out = torch.empty_like(perm)
    _on(perm.device, out=out)
    _index_arg(out, "out", perm.numel())
    ctx = ctx or default_context(perm.device.index)
    _check(_lib().csr_inverse_permutation(ctx.handle, perm.numel(), perm.data_ptr(), out.data_ptr(),
                                          _stream(perm.device)), "csr_inverse_permutation", ctx)
    return out


def gather_values(perm, src, *, out=None, ctx: Optional[Context] = None) -> torch.Tensor:
    """out[k] = src[perm[k]] (per-entry values into a transposed pattern's order)."""
    if perm.dtype != torch.int32 or perm.dim() != 1 or not perm.is_contiguous() or not perm.is_cuda:
        raise ValueError("perm must be a contiguous 1-D int32 GPU tensor")
    _on(perm.device, src=src)
    _entries(src, "src", perm.numel())
    out = _out_entries(out, perm.numel(), perm.device)
    ctx = ctx or default_context(perm.device.index)
    _check(_lib().csr_gather_values(ctx.handle, perm.numel(), perm.data_ptr(), src.data_ptr(), out.data_ptr(),
                                    _stream(perm.device)), "csr_gather_values", ctx)
    return out


def spmm_transposed(At: Transposed, vals, X, *, fused: bool = True, out=None, ctx: Optional[Context] = None,
                    schedule: Optional[CsrSchedule] = None) -> torch.Tensor:
    """A^T X for the transposed pattern At of A, with vals in A's entry order
    (None = 1): one SpMM reading each value through At.perm (fused), or a
    csr_gather_values pass into At's order followed by the SpMM."""
    if vals is None:
        return spmm(At.row_ptr, At.col_idx, None, X, out=out, schedule=schedule, ctx=ctx)
    if fused:
        return spmm(At.row_ptr, At.col_idx, vals, X, val_idx=At.perm, out=out, schedule=schedule, ctx=ctx)
    return spmm(At.row_ptr, At.col_idx, gather_values(At.perm, vals, ctx=ctx), X, out=out, schedule=schedule,
                ctx=ctx)


def spmm_backward(row_ptr, col_idx, vals, X, dY, *, transposed: Optional[Transposed] = None,
                  fused: bool = True, ctx: Optional[Context] = None):
    """Gradients of Y = A X: (d vals, dX) with d vals_e = <dY[row_e], X[col_e]>
    (SDDMM; None when vals is None) and dX = A^T dY (SpMM on the transposed
    pattern, values read through its perm unless ``fused`` is False).
    ``transposed`` (from transpose()) is reused when given."""
    At = transposed or transpose(row_ptr, col_idx, X.shape[0], ctx=ctx)
    dX = spmm_transposed(At, vals, dY, fused=fused, ctx=ctx)
    dvals = None if vals is None else sddmm(row_ptr, col_idx, dY, X, ctx=ctx)
    return dvals, dX


def sddmm_backward(row_ptr, col_idx, U, V, dout, *, transposed: Optional[Transposed] = None,
                   fused: bool = True, ctx: Optional[Context] = None):
    """Gradients of out_e = <U[row_e], V[col_e]>: dU = A_g V and dV = A_g^T U,
    A_g the pattern carrying dout."""
    At = transposed or transpose(row_ptr, col_idx, V.shape[0], ctx=ctx)
    dU = spmm(row_ptr, col_idx, dout, V, ctx=ctx)
    dV = spmm_transposed(At, dout, U, fused=fused, ctx=ctx)
    return dU, dV


def attention_backward(row_ptr, col_idx, edge_scores, node_value, d_out, *, scale: float = 1.0, probs=None,
                       transposed: Optional[Transposed] = None, fused: bool = True, ctx: Optional[Context] = None):
    """Gradients of out = softmax_row(scale * S) V (scores given): returns
    (d edge_scores, d node_value).  P is recomputed by row_softmax unless given;
    dV = P^T d_out and dP = SDDMM(d_out, V); d scores = row_softmax_backward(P,
    dP).  ``fused``: dV and dP in one pass over the transposed pattern
    (spmm_sddmm: each gathered d_out row read once for both, P read through
    the transposed pattern's perm, dP written in the transposed order), dP
    gathered back into A's order through perm's inverse, then the softmax
    backward; otherwise P is gathered into the transposed order, then an SpMM
    and an SDDMM."""
    At = transposed or transpose(row_ptr, col_idx, node_value.shape[0], inverse=fused, ctx=ctx)
    P = probs if probs is not None else row_softmax(row_ptr, edge_scores, scale=scale, ctx=ctx)
    if fused and At.to_t is not None and At.from_t is not None:
        Pt = permute_values(At.to_t, P, ctx=ctx)
        dV, dPt = spmm_sddmm(At.row_ptr, At.col_idx, Pt, d_out, node_value, ctx=ctx)
        dP = permute_values(At.from_t, dPt, out=Pt, ctx=ctx)
        return row_softmax_backward(row_ptr, P, dP, scale=scale, out=dP, ctx=ctx), dV
    if fused:
        inv = At.inv if At.inv is not None else inverse_permutation(At.perm, ctx=ctx)
        dV, dPt = spmm_sddmm(At.row_ptr, At.col_idx, P, d_out, node_value, val_idx=At.perm, ctx=ctx)
        dP = gather_values(inv, dPt, ctx=ctx)
        return row_softmax_backward(row_ptr, P, dP, scale=scale, out=dP, ctx=ctx), dV
    dV = spmm_transposed(At, P, d_out, fused=False, ctx=ctx)
    dP = sddmm(row_ptr, col_idx, d_out, node_value, ctx=ctx)
    dS = row_softmax_backward(row_ptr, P, dP, scale=scale, out=dP, ctx=ctx)
    return dS, dV


def attention_qk_backward(row_ptr, col_idx, Q, K, V, d_out, *, scale: Optional[float] = None,
                          transposed: Optional[Transposed] = None, ctx: Optional[Context] = None):
    """Gradients of the one-head fp32 attention from queries and keys,
    out_i = sum over e of p_e V[col_e] with p the row softmax of
    scale * <Q_i, K[col_e]> (scale 1/sqrt(D) unless given): returns (dQ, dK,
    dV).  The raw scores s_e = <Q_i, K[col_e]> are recomputed by an SDDMM;
    dV and d s come from attention_backward (both products that read d_out in
    one pass over A^T); dQ = dS K (SpMM on A) and dK = dS^T Q (SpMM on A^T
    over dS moved into A^T's order).  ``transposed`` is built with
    permutation plans unless given."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("d_out", d_out)):
        if t.dim() != 2 or t.dtype != torch.float32:
            raise ValueError(f"{name} must be 2-D float32 (one head)")
    if Q.shape[0] != n_rows or d_out.shape[0] != n_rows or K.shape[0] != V.shape[0] or K.shape[1] != Q.shape[1] \
            or d_out.shape[1] != V.shape[1]:
        raise ValueError("Q, d_out: [n_rows, ...]; K, V: [n_cols, ...]; K as wide as Q, d_out as wide as V")
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[1])
    At = transposed or transpose(row_ptr, col_idx, K.shape[0], plans=True, ctx=ctx)
    S = sddmm(row_ptr, col_idx, Q, K, ctx=ctx)
    dS, dV = attention_backward(row_ptr, col_idx, S, V, d_out, scale=scale, transposed=At, ctx=ctx)
    dQ = spmm(row_ptr, col_idx, dS, K, ctx=ctx)
    if At.to_t is not None:
        dK = spmm(At.row_ptr, At.col_idx, permute_values(At.to_t, dS, out=S, ctx=ctx), Q, ctx=ctx)
    else:
        dK = spmm(At.row_ptr, At.col_idx, dS, Q, val_idx=At.perm, ctx=ctx)
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# column-part segment format
# ---------------------------------------------------------------------------

class Hybrid:
    """A column-part segment format of a CSR pattern (see hybrid_format): the
    device arrays and the csr_hybrid_t that describes them.  seg_ptr, seg_row
    and row_seg are views of their first n_seg (+1) entries."""

    def __init__(self, desc: CsrHybrid, arrays: dict):
        self.desc = desc
        self._arrays = arrays  # keeps the device memory alive
        n = desc.n_seg
        self.n_rows, self.n_cols, self.nnz = desc.n_rows, desc.n_cols, desc.nnz
        self.parts, self.part_cols, self.n_seg = desc.parts, desc.part_cols, n
        self.whole_below = desc.whole_below
        self.perm, self.col_idx = arrays["perm"], arrays["col_idx"]
        self.seg_ptr = arrays["seg_ptr"][:n + 1]
        self.seg_row = arrays["seg_row"][:n]
        self.row_seg_ptr = arrays["row_seg_ptr"]
        self.row_seg = arrays["row_seg"][:n]

    def __repr__(self):
        return (f"Hybrid(n_rows={self.n_rows}, n_cols={self.n_cols}, nnz={self.nnz}, parts={self.parts}, "
                f"part_cols={self.part_cols}, whole_below={self.whole_below}, n_seg={self.n_seg})")


def hybrid_plan(problem: CsrProblem, histogram=None):
    """(parts, whole_below) of the column-part segment format expected to be
    fastest for this problem (parts 1: use the plain CSR path)."""
    h = None if histogram is None else (ctypes.c_int64 * 67)(*[int(v) for v in histogram])
    parts, whole = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib().csr_hybrid_plan(None, ctypes.byref(problem), h, ctypes.byref(parts), ctypes.byref(whole)),
           "csr_hybrid_plan")
    return parts.value, whole.value


def hybrid_parts(problem: CsrProblem, histogram=None) -> int:
    """The parts of hybrid_plan."""
    return hybrid_plan(problem, histogram)[0]


def hybrid_format(row_ptr, col_idx, n_cols: int, parts: int, *, whole_below: int = 0,
                  ctx: Optional[Context] = None) -> Hybrid:
    """Builds the column-part segment format of (row_ptr, col_idx) with
    ``parts`` column parts (a power of two from 1 to 256); rows with fewer
    than ``whole_below`` entries stay whole (one segment after all parts)."""
    n_rows, nnz = _pattern(row_ptr, col_idx)
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    lib = _lib()
    cap = ctypes.c_int64()
    _check(lib.csr_hybrid_capacity(n_rows, nnz, parts, ctypes.byref(cap)), "csr_hybrid_capacity")
    nbytes = ctypes.c_size_t()
    _check(lib.csr_hybrid_build_workspace_size(ctx.handle, n_rows, nnz, parts, ctypes.byref(nbytes)),
           "csr_hybrid_build_workspace_size", ctx)
    ws = _workspace(device, nbytes.value)

    def i32(n):
        return torch.empty(max(n, 1), dtype=torch.int32, device=device)

    arrays = {"perm": i32(nnz)[:nnz], "col_idx": i32(nnz)[:nnz], "seg_ptr": i32(cap.value + 1),
              "seg_row": i32(cap.value), "row_seg_ptr": i32(n_rows + 1), "row_seg": i32(cap.value)}
    h = CsrHybrid()
    h.n_rows, h.n_cols, h.nnz, h.parts, h.seg_cap = n_rows, n_cols, nnz, parts, cap.value
    h.whole_below = whole_below
    for k, t in arrays.items():
        setattr(h, k, t.data_ptr())
    _check(lib.csr_hybrid_build(ctx.handle, row_ptr.data_ptr(), col_idx.data_ptr(), ctypes.byref(h), ws.data_ptr(),
                                nbytes.value, _stream(device)), "csr_hybrid_build", ctx)
    return Hybrid(h, arrays)


def hybrid_values(h: Hybrid, vals, *, out=None, ctx: Optional[Context] = None) -> torch.Tensor:
    """Per-entry values moved into the format's entry order (vals[perm])."""
    return gather_values(h.perm, vals, out=out, ctx=ctx)


def hybrid_problem(h: Hybrid, op: str, *operands) -> CsrProblem:
    """The plain problem of the segment product ('spmm': vals, X; 'sddmm': U, V),
    for candidates() / default_schedule(): its schedules are the ones that
    hybrid_spmm / hybrid_sddmm accept."""
    if op == "spmm":
        vals, X = operands
        p = _problem(_ffi.OP_SPMM, h.seg_ptr, h.col_idx, vals, X, None, None, n_cols=X.shape[0], width=X.shape[1],
                     ld_b=_dense(X, "X", (torch.float32, torch.bfloat16)), ld_out=X.shape[1], dtype=_dtype_code(X, "X"))
        p.out = 256  # stands for the partial rows, which sit 256-byte aligned in the workspace
        return p
    if op == "sddmm":
        U, V = operands
        return _sddmm_problem(h.seg_ptr, h.col_idx, U, V, None)
    raise ValueError(op)


def _hybrid_run(h, op, width, dtype, schedule, ctx, device, call, workspace=None):
    ctx = ctx or default_context(device.index)
    lib = _lib()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_hybrid_workspace_size(ctx.handle, ctypes.byref(h.desc), op, width, dtype, _sched_arg(schedule),
                                         ctypes.byref(nbytes)), "csr_hybrid_workspace_size", ctx)
    ws = _workspace(device, nbytes.value, workspace)
    _check(call(ctx, ws, nbytes.value, _stream(device)), "csr hybrid call", ctx)


def hybrid_select(h: Hybrid, op: str, *operands, mode: str = "auto", out=None, ctx: Optional[Context] = None):
    """Selects the segment product's schedule for a call over the format
    ('spmm': format-order vals or None, X; 'sddmm': U, V); returns
    (schedule, signature).  Probes run on the given operands (SDDMM: they
    write ``out``)."""
    a, b = operands
    device = b.device
    ctx = ctx or default_context(device.index)
    lib = _lib()
    call = CsrProblem()
    call.op = _ffi.OP_SPMM if op == "spmm" else _ffi.OP_SDDMM if op == "sddmm" else -1
    if call.op < 0:
        raise ValueError(op)
    call.width = b.shape[1]
    call.b, call.ld_b = b.data_ptr(), _dense(b, "X" if op == "spmm" else "V", (torch.float32, torch.bfloat16))
    call.dtype = _dtype_code(b, "X" if op == "spmm" else "V")
    if op == "spmm":
        call.a = _ptr(a)
    else:
        call.a, call.ld_a = a.data_ptr(), _dense(a, "U", (torch.float32, torch.bfloat16))
        if a.dtype != b.dtype:
            raise TypeError("U and V must have one dtype")
        out = out if out is not None else torch.empty(h.nnz, dtype=torch.float32, device=device)
        call.out = out.data_ptr()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_hybrid_workspace_size(ctx.handle, ctypes.byref(h.desc), call.op, call.width, call.dtype, None,
                                         ctypes.byref(nbytes)), "csr_hybrid_workspace_size", ctx)
    ws = _workspace(device, nbytes.value)
    call.workspace, call.workspace_bytes, call.stream = ws.data_ptr(), nbytes.value, _stream(device)
    s, sig = CsrSchedule(), ctypes.c_uint64()
    _check(lib.csr_hybrid_select(ctx.handle, ctypes.byref(h.desc), ctypes.byref(call), _ffi.SELECT_MODES[mode],
                                 ctypes.byref(s), ctypes.byref(sig)), "csr_hybrid_select", ctx)
    return s, sig.value


def hybrid_spmm(h: Hybrid, vals, X, *, out=None, schedule: Optional[CsrSchedule] = None,
                ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = A X over the format; ``vals`` in the format's entry order
    (hybrid_values) or None for all ones."""
    _on(h.perm.device, vals=vals, X=X)
    _rows(X, "X", h.n_cols, dtype=(torch.float32, torch.bfloat16))
    ldx = _dense(X, "X", (torch.float32, torch.bfloat16))
    xd = _dtype_code(X, "X")
    out = _out_rows(out, h.n_rows, X.shape[1], X.device)
    ldy = _dense(out, "out", torch.float32)
    if vals is not None:
        _flat_f32(vals, "vals", h.nnz)

    def call(ctx, ws, nb, st):
        return _lib().csr_hybrid_spmm(ctx.handle, ctypes.byref(h.desc), _ptr(vals), X.data_ptr(), xd, X.shape[1],
                                      ldx, out.data_ptr(), ldy, _sched_arg(schedule), ws.data_ptr(), nb, st)

    _hybrid_run(h, _ffi.OP_SPMM, X.shape[1], xd, schedule, ctx, X.device, call, workspace)
    return out


def hybrid_sddmm(h: Hybrid, U, V, *, out=None, schedule: Optional[CsrSchedule] = None,
                 ctx: Optional[Context] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[e] = <U[row(e)], V[col(e)]> over the format, in the original entry order."""
    _on(h.perm.device, U=U, V=V)
    _rows(U, "U", h.n_rows, dtype=(torch.float32, torch.bfloat16))
    _rows(V, "V", h.n_cols, U.shape[1], dtype=U.dtype)
    ldu = _dense(U, "U", (torch.float32, torch.bfloat16))
    ldv = _dense(V, "V", (torch.float32, torch.bfloat16))
    dt = _dtype_code(U, "U")
    out = _out_entries(out, h.nnz, U.device)

    def call(ctx, ws, nb, st):
        return _lib().csr_hybrid_sddmm(ctx.handle, ctypes.byref(h.desc), U.data_ptr(), ldu, V.data_ptr(), ldv, dt,
                                       U.shape[1], out.data_ptr(), _sched_arg(schedule), ws.data_ptr(), nb, st)

    _hybrid_run(h, _ffi.OP_SDDMM, U.shape[1], dt, schedule, ctx, U.device, call, workspace)
    return out


# ---------------------------------------------------------------------------
# planned products: the library chooses layout (plain CSR or the column-part
# segment format at some part count and whole-row threshold) and schedule
# together, and caches the choice
# ---------------------------------------------------------------------------

class Plan:
    """A CSR matrix prepared for one SpMM or SDDMM (csr_plan_t): the chosen
    layout (the plain pattern, the column-part format, or the degree classes)
    and schedule, the plan memory that holds its arrays, and the tensors it
    refers to (kept alive with it)."""

    def __init__(self, desc: CsrPlan, mem, keep):
        self.desc = desc
        self._mem = mem
        self._keep = keep

    @property
    def op(self):
        return {_ffi.OP_SPMM: "spmm", _ffi.OP_SDDMM: "sddmm"}[self.desc.op]

    @property
    def parts(self):
        return self.desc.parts

    @property
    def whole_below(self):
        return self.desc.whole_below

    @property
    def schedule(self) -> CsrSchedule:
        return CsrSchedule.from_buffer_copy(bytes(self.desc.sched))

    @property
    def signature(self) -> int:
        return self.desc.signature

    @property
    def layout(self) -> str:
        """'plain' (the caller's CSR), 'format' (column parts) or 'classes' (degree classes)."""
        return {0: "classes", 1: "plain"}.get(self.desc.parts, "format")

    @property
    def n_seg(self) -> int:
        return self.desc.fmt.n_seg if self.desc.parts > 1 else 0

    @property
    def workspace_bytes(self) -> int:
        return self.desc.workspace_bytes

    def choice(self):
        """(parts, whole_below, schedule as a dict): the plan's joint choice."""
        return self.parts, self.whole_below, self.schedule.as_dict()

    def __repr__(self):
        if self.desc.parts == 0:
            b = self.desc.bkt
            shape = f"short_below={b.short_below}, n_short={b.n_short}, n_slots={b.n_slots}, nnz_long={b.nnz_long}"
        else:
            shape = f"parts={self.parts}, whole_below={self.whole_below}, n_seg={self.n_seg}"
        return f"Plan({self.op}, {self.layout}, {shape}, {self.schedule}, probe_ms={self.desc.probe_ms:.3f})"


def plan(op: str, row_ptr, col_idx, *operands, mode: str = "auto", layout=None,
         schedule: Optional[CsrSchedule] = None, out=None, ctx: Optional[Context] = None) -> Plan:
    """Plans a product ('spmm': vals or None, X; 'sddmm': U, V): the library
    chooses the layout and the schedule together by its cost model and
    micro-probes on these operands (the probes write ``out``), or replays the
    cached choice.  With ``layout`` = (parts, whole_below) the plan takes that
    layout (parts 1 the plain pattern, 2 .. 256 the column-part format, 0 the
    degree classes with short threshold whole_below) and ``schedule`` for its
    product, or the selector's schedule when none is given (csr_plan_build;
    nothing cached).  Synchronous."""
    if op not in ("spmm", "sddmm"):
        raise ValueError("plans serve 'spmm' and 'sddmm'")
    if schedule is not None and layout is None:
        raise ValueError("a schedule is given with a layout")
    p, out = make_problem(op, row_ptr, col_idx, *operands, out=out)
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    lib = _lib()
    head = _workspace(device, 1024)
    p.workspace, p.workspace_bytes, p.stream = head.data_ptr(), 1024, _stream(device)
    mem_bytes, ws_bytes = ctypes.c_size_t(), ctypes.c_size_t()
    if layout is None:
        _check(lib.csr_plan_size(ctx.handle, ctypes.byref(p), ctypes.byref(mem_bytes), ctypes.byref(ws_bytes)),
               "csr_plan_size", ctx)
    else:
        parts, whole = (int(v) for v in layout)
        _check(lib.csr_plan_layout_size(ctx.handle, ctypes.byref(p), parts, whole, ctypes.byref(mem_bytes),
                                        ctypes.byref(ws_bytes)), "csr_plan_layout_size", ctx)
    mem = torch.empty(mem_bytes.value + 256, dtype=torch.uint8, device=device)
    off = (-mem.data_ptr()) % 256
    ws = _workspace(device, ws_bytes.value)
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws_bytes.value
    desc = CsrPlan()
    if layout is None:
        _check(lib.csr_plan_create(ctx.handle, ctypes.byref(p), _ffi.SELECT_MODES[mode], mem.data_ptr() + off,
                                   mem_bytes.value, ctypes.byref(desc)), "csr_plan_create", ctx)
    else:
        _check(lib.csr_plan_build(ctx.handle, ctypes.byref(p), parts, whole, _sched_arg(schedule),
                                  mem.data_ptr() + off, mem_bytes.value, ctypes.byref(desc)), "csr_plan_build", ctx)
    keep = (row_ptr, col_idx) + tuple(t for t in operands if t is not None)
    return Plan(desc, mem, keep)


def plan_spmm(pl: Plan, X, *, vals=None, out=None, ctx: Optional[Context] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = A X with a plan of 'spmm'; ``vals`` (original entry order), when
    given, are this call's values instead of the plan's (for this call only)."""
    if pl.desc.op != _ffi.OP_SPMM:
        raise ValueError("not a plan of 'spmm'")
    _rows(X, "X", pl.desc.n_cols, pl.desc.width, dtype=(torch.float32, torch.bfloat16))
    ldx = _dense(X, "X", (torch.float32, torch.bfloat16))
    if _dtype_code(X, "X") != pl.desc.dtype:
        raise TypeError("X's dtype is not the plan's")
    if vals is not None:
        _entries(vals, "vals", pl.desc.nnz)
    out = _out_rows(out, pl.desc.n_rows, pl.desc.width, X.device)
    ldy = _dense(out, "out", torch.float32)
    ctx = ctx or default_context(X.device.index)
    ws = _workspace(X.device, pl.desc.workspace_bytes, workspace)
    _check(_lib().csr_plan_spmm(ctx.handle, ctypes.byref(pl.desc), _ptr(vals), X.data_ptr(), ldx, out.data_ptr(), ldy,
                                ws.data_ptr(), pl.desc.workspace_bytes, _stream(X.device)), "csr_plan_spmm", ctx)
    return out


def plan_sddmm(pl: Plan, U, V, *, out=None, ctx: Optional[Context] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[e] = <U[row_e], V[col_e]> (original entry order) with a plan of 'sddmm'."""
    if pl.desc.op != _ffi.OP_SDDMM:
        raise ValueError("not a plan of 'sddmm'")
    _rows(U, "U", pl.desc.n_rows, pl.desc.width, dtype=(torch.float32, torch.bfloat16))
    _rows(V, "V", pl.desc.n_cols, pl.desc.width, dtype=U.dtype)
    if _dtype_code(U, "U") != pl.desc.dtype:
        raise TypeError("U's dtype is not the plan's")
    ldu, ldv = _dense(U, "U", U.dtype), _dense(V, "V", V.dtype)
    out = _out_entries(out, pl.desc.nnz, U.device)
    ctx = ctx or default_context(U.device.index)
    ws = _workspace(U.device, pl.desc.workspace_bytes, workspace)
    _check(_lib().csr_plan_sddmm(ctx.handle, ctypes.byref(pl.desc), U.data_ptr(), ldu, V.data_ptr(), ldv,
                                 out.data_ptr(), ws.data_ptr(), pl.desc.workspace_bytes, _stream(U.device)),
           "csr_plan_sddmm", ctx)
    return out


def make_problem(op: str, row_ptr, col_idx, *operands, out=None, scale: float = 1.0, val_idx=None,
                 z_idx=None) -> CsrProblem:
    """The csr_problem_t of a call, for select() / workspace_size() /
    default_schedule(): op is 'spmm' (vals, X; val_idx: the value index of
    csr_spmm_perm), 'spmm_sddmm' (vals, X, U; val_idx, z_idx), 'sddmm' (U, V), 'attention' (edge_scores, node_value),
    'mha' (Q, K, V) or 'attention_qk' (Q, K, V: the problem that
    csr_attention runs for them)."""
    _pattern(row_ptr, row_ptr if col_idx is None else col_idx)
    n_rows = row_ptr.numel() - 1
    if val_idx is not None and op not in ("spmm", "spmm_sddmm"):
        raise ValueError("val_idx serves 'spmm' and 'spmm_sddmm'")
    if z_idx is not None and op != "spmm_sddmm":
        raise ValueError("z_idx serves 'spmm_sddmm'")
    if op == "spmm":
        vals, X = operands
        out = out if out is not None else torch.empty((n_rows, X.shape[1]), dtype=torch.float32, device=X.device)
        p = _spmm_problem(row_ptr, col_idx, vals, X, out)
        if val_idx is not None:
            p.a_idx = val_idx.data_ptr()
        return p, out
    if op == "spmm_sddmm":
        vals, X, U = operands
        out = out if out is not None else torch.empty((n_rows, X.shape[1]), dtype=torch.float32, device=X.device)
        z = torch.empty(col_idx.numel(), dtype=torch.float32, device=X.device)
        return _spmm_sddmm_problem(row_ptr, col_idx, vals, X, U, out, z, val_idx, z_idx), out
    if op == "sddmm":
        U, V = operands
        out = out if out is not None else torch.empty(col_idx.numel(), dtype=torch.float32, device=U.device)
        return _sddmm_problem(row_ptr, col_idx, U, V, out), out
    if op == "attention":
        s, nv = operands
        out = out if out is not None else torch.empty((n_rows, nv.shape[1]), dtype=torch.float32, device=nv.device)
        return _attention_problem(row_ptr, col_idx, s, nv, out, scale), out
    if op == "row_softmax":
        (scores,) = operands
        out = out if out is not None else torch.empty_like(scores)
        return _softmax_problem(row_ptr, scores, out, scale), out
    if op == "row_softmax_backward":
        probs, grad = operands
        out = out if out is not None else torch.empty_like(probs)
        return _softmax_bwd_problem(row_ptr, probs, grad, out, scale), out
    if op == "mha":
        Q, K, V = operands
        out = out if out is not None else torch.empty((n_rows,) + tuple(Q.shape[1:]), dtype=torch.float32,
                                                       device=Q.device)
        return _mha_problem(row_ptr, col_idx, Q, K, V, out, scale), out
    if op == "attention_qk":
        Q, K, V = operands
        out = out if out is not None else torch.empty(tuple(Q.shape), dtype=torch.float32, device=Q.device)
        return _qk_problem(row_ptr, col_idx, Q, K, V, out, None, scale)[0], out
    raise ValueError(op)


def select(op: str, row_ptr, col_idx, *operands, mode: str = "auto", scale: float = 1.0, out=None,
           val_idx=None, z_idx=None, ctx: Optional[Context] = None):
    """Runs the selector for a call; returns (schedule, signature).  With
    mode 'auto' or 'probe' the candidates run on the given operands and write
    ``out``."""
    p, out = make_problem(op, row_ptr, col_idx, *operands, out=out, scale=scale, val_idx=val_idx, z_idx=z_idx)
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    lib = _lib()
    nbytes = ctypes.c_size_t()
    _check(lib.csr_workspace_size(ctx.handle, ctypes.byref(p), None, ctypes.byref(nbytes)), "csr_workspace_size", ctx)
    ws = _workspace(device, nbytes.value)
    p.workspace, p.workspace_bytes, p.stream = ws.data_ptr(), nbytes.value, _stream(device)
    s, sig = CsrSchedule(), ctypes.c_uint64()
    _check(lib.csr_select(ctx.handle, ctypes.byref(p), _ffi.SELECT_MODES[mode], ctypes.byref(s), ctypes.byref(sig)),
           "csr_select", ctx)
    return s, sig.value


def default_schedule(problem: CsrProblem) -> CsrSchedule:
    s = CsrSchedule()
    _check(_lib().csr_default_schedule(None, ctypes.byref(problem), ctypes.byref(s)), "csr_default_schedule")
    return s


def candidates(problem: CsrProblem, histogram=None):
    """The selector's candidate schedules for a problem (and degree histogram)."""
    h = None if histogram is None else (ctypes.c_int64 * 67)(*[int(v) for v in histogram])
    n = ctypes.c_int32()
    _check(_lib().csr_candidates(None, ctypes.byref(problem), h, None, 0, ctypes.byref(n)), "csr_candidates")
    arr = (CsrSchedule * max(1, n.value))()
    _check(_lib().csr_candidates(None, ctypes.byref(problem), h, arr, n.value, ctypes.byref(n)), "csr_candidates")
    return [CsrSchedule.from_buffer_copy(bytes(arr[i])) for i in range(n.value)]


def workspace_size(problem: CsrProblem, schedule: Optional[CsrSchedule] = None) -> int:
    n = ctypes.c_size_t()
    _check(_lib().csr_workspace_size(None, ctypes.byref(problem), _sched_arg(schedule), ctypes.byref(n)),
           "csr_workspace_size")
    return n.value


def signature(problem: CsrProblem, histogram, ctx: Optional[Context] = None) -> int:
    h = (ctypes.c_int64 * 67)(*[int(v) for v in histogram])
    out = ctypes.c_uint64()
    _check(_lib().csr_signature(ctx.handle if ctx else None, ctypes.byref(problem), h, ctypes.byref(out)),
           "csr_signature")
    return out.value


def degree_histogram(row_ptr, *, ctx: Optional[Context] = None):
    """(counts[33], degree sums[33], max degree) of a device CSR row_ptr."""
    _pattern(row_ptr, row_ptr)
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    out = (ctypes.c_int64 * 67)()
    ws = _workspace(device, 1024)
    _check(_lib().csr_degree_histogram(ctx.handle, row_ptr.numel() - 1, row_ptr.data_ptr(), out, ws.data_ptr(),
                                       1024, _stream(device)), "csr_degree_histogram", ctx)
    vals = list(out)
    return vals[:33], vals[33:66], vals[66]


def merge_path_partition(row_ptr, nnz: int, items_per_chunk: int, *, ctx: Optional[Context] = None):
    """Device int32 tensor [n_chunks + 1, 2] of (rows ended, entries consumed)."""
    device = row_ptr.device
    ctx = ctx or default_context(device.index)
    n_rows = row_ptr.numel() - 1
    n_chunks = max(1, -(-(n_rows + nnz) // items_per_chunk))
    coords = torch.empty((n_chunks + 1, 2), dtype=torch.int32, device=device)
    _check(_lib().csr_merge_path_partition(ctx.handle, n_rows, nnz, row_ptr.data_ptr(), items_per_chunk,
                                           coords.data_ptr(), _stream(device)), "csr_merge_path_partition", ctx)
    return coords
