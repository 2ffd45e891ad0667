"""ctypes declarations of the C ABI in include/csrsa.h."""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# CSRSA_LIB names another build of the library (side-by-side comparisons);
# by default the in-tree build is loaded.
LIB_PATH = os.environ.get("CSRSA_LIB") or os.path.join(PKG, "libcsrsa.so")

# status codes
CSR_OK = 0
STATUS = {
    0: "CSR_OK", -1: "CSR_ERR_NULL", -2: "CSR_ERR_SHAPE", -3: "CSR_ERR_DTYPE", -4: "CSR_ERR_ALIGN",
    -5: "CSR_ERR_WORKSPACE", -6: "CSR_ERR_INVALID_CSR", -7: "CSR_ERR_SCHEDULE", -8: "CSR_ERR_NO_CACHE_ENTRY",
    -9: "CSR_ERR_CACHE_IO", -10: "CSR_ERR_HIP", -11: "CSR_ERR_DEVICE", -12: "CSR_ERR_INTERNAL",
}
CSR_ERR_NO_CACHE_ENTRY = -8

OP_SPMM, OP_SDDMM, OP_ATTENTION, OP_MHA, OP_ROW_SOFTMAX, OP_SOFTMAX_BWD, OP_ATTENTION_QK, OP_SPMM_SDDMM = \
    1, 2, 3, 4, 5, 6, 7, 8
DTYPE_F32, DTYPE_BF16 = 0, 1
MAP_ROWGROUP, MAP_MERGEPATH, MAP_SEGSCAN = 1, 2, 3
SCHED_WIDE = 1  # schedule flag: 16-byte lanes over 4-byte aligned rows (SpMM, row-group)
CTX_VALIDATE, CTX_NO_PROBE = 1, 2
SELECT_MODES = {"auto": 0, "replay": 1, "probe": 2, "estimate": 3}
SCHEDULE_VERSION = 1
NOALLOC_SCRATCH_BYTES = 32 << 20  # CSR_NOALLOC_SCRATCH_BYTES

# Every symbol the header declares.
EXPORTS = (
    "csr_context_create", "csr_context_destroy", "csr_status_string", "csr_last_error",
    "csr_spmm", "csr_spmm_perm", "csr_spmm_sddmm", "csr_spmm_noalloc", "csr_sddmm", "csr_attention", "csr_mha_attention", "csr_row_softmax",
    "csr_row_softmax_backward", "csr_transpose_workspace_size", "csr_transpose",
    "csr_gather_values", "csr_inverse_permutation", "csr_permutation_plan_workspace_size", "csr_permutation_plan",
    "csr_permute_values",
    "csr_select", "csr_default_schedule", "csr_candidates", "csr_workspace_size", "csr_cache_flush",
    "csr_cache_info", "csr_cache_lookup", "csr_cache_store",
    "csr_degree_histogram", "csr_merge_path_partition", "csr_signature",
    "csr_hybrid_plan", "csr_hybrid_parts", "csr_hybrid_capacity", "csr_hybrid_build_workspace_size", "csr_hybrid_build", "csr_hybrid_workspace_size",
    "csr_hybrid_spmm", "csr_hybrid_sddmm", "csr_hybrid_select",
    "csr_plan_size", "csr_plan_create", "csr_plan_layout_size", "csr_plan_build", "csr_plan_spmm", "csr_plan_sddmm",
)


class CsrSchedule(ctypes.Structure):
    _fields_ = [
        ("version", ctypes.c_int32),
        ("op", ctypes.c_int32),
        ("mapping", ctypes.c_int32),
        ("vec", ctypes.c_int32),
        ("group_lanes", ctypes.c_int32),
        ("passes", ctypes.c_int32),
        ("chunk_items", ctypes.c_int32),
        ("long_row", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 7),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}

    def key(self) -> bytes:
        return bytes(self)

    def __repr__(self):
        d = self.as_dict()
        return "CsrSchedule(" + ", ".join(f"{k}={v}" for k, v in d.items()) + ")"

    def __eq__(self, other):
        return isinstance(other, CsrSchedule) and bytes(self) == bytes(other)

    def __hash__(self):
        return hash(bytes(self))


class CsrProblem(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("n_cols", ctypes.c_int64),
        ("nnz", ctypes.c_int64),
        ("width", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("ld_a", ctypes.c_int64),
        ("ld_b", ctypes.c_int64),
        ("ld_out", ctypes.c_int64),
        ("row_ptr", ctypes.c_void_p),
        ("col_idx", ctypes.c_void_p),
        ("a", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("c", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("pad_", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("ld_c", ctypes.c_int64),
        ("probs", ctypes.c_void_p),
        ("probs_stride", ctypes.c_int64),
        ("a_idx", ctypes.c_void_p),
        ("out2", ctypes.c_void_p),
        ("out2_idx", ctypes.c_void_p),
    ]


assert ctypes.sizeof(CsrSchedule) == 64


class CsrHybrid(ctypes.Structure):
    """csr_hybrid_t: a column-part segment format (device arrays owned by the caller)."""
    _fields_ = [
        ("n_rows", ctypes.c_int64),
        ("n_cols", ctypes.c_int64),
        ("nnz", ctypes.c_int64),
        ("parts", ctypes.c_int32),
        ("part_cols", ctypes.c_int32),
        ("whole_below", ctypes.c_int32),
        ("reserved_", ctypes.c_int32),
        ("seg_cap", ctypes.c_int64),
        ("n_seg", ctypes.c_int64),
        ("perm", ctypes.c_void_p),
        ("col_idx", ctypes.c_void_p),
        ("seg_ptr", ctypes.c_void_p),
        ("seg_row", ctypes.c_void_p),
        ("row_seg_ptr", ctypes.c_void_p),
        ("row_seg", ctypes.c_void_p),
    ]


assert ctypes.sizeof(CsrHybrid) == 104

PLAN_VERSION = 1


class CsrBucket(ctypes.Structure):
    """csr_bucket_t: degree classes (short rows packed slot-major by class, the
    other rows as a CSR of their own), arrays in the plan memory."""
    _fields_ = [
        ("short_below", ctypes.c_int32),
        ("n_classes", ctypes.c_int32),
        ("n_short", ctypes.c_int64),
        ("n_slots", ctypes.c_int64),
        ("nnz_long", ctypes.c_int64),
        ("class_rows", ctypes.c_int64 * 6),
        ("rows", ctypes.c_void_p),
        ("slot_col", ctypes.c_void_p),
        ("slot_pos", ctypes.c_void_p),
        ("slot_val", ctypes.c_void_p),
        ("long_row_ptr", ctypes.c_void_p),
        ("long_col", ctypes.c_void_p),
        ("long_pos", ctypes.c_void_p),
        ("long_val", ctypes.c_void_p),
    ]


class CsrPlan(ctypes.Structure):
    """csr_plan_t: a CSR matrix prepared for one SpMM or SDDMM (layout and schedule)."""
    _fields_ = [
        ("version", ctypes.c_int32),
        ("op", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("parts", ctypes.c_int32),
        ("whole_below", ctypes.c_int32),
        ("reserved_", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("n_cols", ctypes.c_int64),
        ("nnz", ctypes.c_int64),
        ("width", ctypes.c_int64),
        ("signature", ctypes.c_uint64),
        ("sched", CsrSchedule),
        ("fmt", CsrHybrid),
        ("bkt", CsrBucket),
        ("row_ptr", ctypes.c_void_p),
        ("col_idx", ctypes.c_void_p),
        ("vals", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("probe_ms", ctypes.c_double),
    ]


assert ctypes.sizeof(CsrBucket) == 144
assert ctypes.sizeof(CsrPlan) == 416


class CsrError(RuntimeError):
    def __init__(self, code: int, where: str, message: str = ""):
        self.code = code
        name = STATUS.get(code, str(code))
        super().__init__(f"{where}: {name}" + (f" ({message})" if message else ""))


_lib = None


def load() -> ctypes.CDLL:
    """Loads libcsrsa.so; raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python csr_sparse_attention_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, U32, F, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                               ctypes.c_float, ctypes.c_size_t)
    SP, PP, HP = ctypes.POINTER(CsrSchedule), ctypes.POINTER(CsrProblem), ctypes.POINTER(CsrHybrid)
    PLP = ctypes.POINTER(CsrPlan)
    sig = {
        "csr_context_create": [ctypes.POINTER(P), ctypes.c_int, ctypes.c_char_p, U32],
        "csr_context_destroy": [P],
        "csr_status_string": [ctypes.c_int],
        "csr_last_error": [P],
        "csr_spmm": [P, I64, I64, I64, P, P, P, P, I32, I64, I64, P, I64, SP, P, SZ, P],
        "csr_spmm_noalloc": [P, I64, I64, I64, P, P, P, P, I32, I64, I64, P, I64, SP, P],
        "csr_spmm_perm": [P, I64, I64, I64, P, P, P, P, P, I32, I64, I64, P, I64, SP, P, SZ, P],
        "csr_spmm_sddmm": [P, I64, I64, I64, P, P, P, P, P, I64, I64, P, I64, P, I64, P, P, SP, P, SZ, P],
        "csr_sddmm": [P, I64, I64, I64, P, P, P, I64, P, I64, I32, I64, P, SP, P, SZ, P],
        "csr_attention": [P, I64, I64, I64, P, P, P, P, P, P, I32, I32, I64, I64, F, P, I64, P, SP, P, SZ, P],
        "csr_mha_attention": [P, I64, I64, I64, P, P, P, P, P, I32, I32, F, P, P, SP, P, SZ, P],
        "csr_row_softmax": [P, I64, I64, P, P, F, P, SP, P, SZ, P],
        "csr_row_softmax_backward": [P, I64, I64, P, P, P, F, P, SP, P, SZ, P],
        "csr_transpose_workspace_size": [P, I64, I64, I64, ctypes.POINTER(SZ)],
        "csr_transpose": [P, I64, I64, I64, P, P, P, P, P, P, SZ, P],
        "csr_gather_values": [P, I64, P, P, P, P],
        "csr_inverse_permutation": [P, I64, P, P, P],
        "csr_permutation_plan_workspace_size": [P, I64, ctypes.POINTER(SZ)],
        "csr_permutation_plan": [P, I64, P, I32, P, P, P, SZ, P],
        "csr_permute_values": [P, I64, P, P, P, P, P, P],
        "csr_select": [P, PP, U32, SP, ctypes.POINTER(ctypes.c_uint64)],
        "csr_default_schedule": [P, PP, SP],
        "csr_candidates": [P, PP, ctypes.POINTER(I64), SP, I32, ctypes.POINTER(I32)],
        "csr_workspace_size": [P, PP, SP, ctypes.POINTER(SZ)],
        "csr_cache_flush": [P],
        "csr_cache_info": [P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "csr_cache_lookup": [P, ctypes.c_uint64, SP],
        "csr_cache_store": [P, ctypes.c_uint64, SP],
        "csr_degree_histogram": [P, I64, P, ctypes.POINTER(I64), P, SZ, P],
        "csr_merge_path_partition": [P, I64, I64, P, I32, P, P],
        "csr_signature": [P, PP, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_uint64)],
        "csr_hybrid_plan": [P, PP, ctypes.POINTER(I64), ctypes.POINTER(I32), ctypes.POINTER(I32)],
        "csr_hybrid_parts": [P, PP, ctypes.POINTER(I64), ctypes.POINTER(I32)],
        "csr_hybrid_capacity": [I64, I64, I32, ctypes.POINTER(I64)],
        "csr_hybrid_build_workspace_size": [P, I64, I64, I32, ctypes.POINTER(SZ)],
        "csr_hybrid_build": [P, P, P, HP, P, SZ, P],
        "csr_hybrid_workspace_size": [P, HP, I32, I64, I32, SP, ctypes.POINTER(SZ)],
        "csr_hybrid_spmm": [P, HP, P, P, I32, I64, I64, P, I64, SP, P, SZ, P],
        "csr_hybrid_sddmm": [P, HP, P, I64, P, I64, I32, I64, P, SP, P, SZ, P],
        "csr_hybrid_select": [P, HP, PP, U32, SP, ctypes.POINTER(ctypes.c_uint64)],
        "csr_plan_size": [P, PP, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "csr_plan_create": [P, PP, U32, P, SZ, PLP],
        "csr_plan_layout_size": [P, PP, I32, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "csr_plan_build": [P, PP, I32, I32, SP, P, SZ, PLP],
        "csr_plan_spmm": [P, PLP, P, P, I64, P, I64, P, SZ, P],
        "csr_plan_sddmm": [P, PLP, P, I64, P, I64, P, P, SZ, P],
    }
    for name, argtypes in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name in ("csr_status_string", "csr_last_error") else ctypes.c_int
    _lib = lib
    return lib
