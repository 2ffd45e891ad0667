"""MI355X-native CSR sparse aggregation: SpMM, SDDMM and fused CSR softmax
attention with an input-aware schedule selector and a persistent cache.

The computation lives in ``libcsrsa.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/csrsa.h``); this package is a thin ctypes
binding over it and raises ImportError when the library has not been built.
"""

# torch first: its bundled HIP runtime carries the same soname as ROCm's, so
# loading it before libcsrsa.so makes the library bind to that one runtime
# (torch's streams and allocations are then valid in library calls); the
# other order would put two HIP runtimes in the process.
import torch  # noqa: F401

from ._ffi import (  # noqa: F401,E402
    OP_SOFTMAX_BWD,
    CsrError,
    CsrHybrid,
    CsrPlan,
    CsrProblem,
    CsrSchedule,
    EXPORTS,
    LIB_PATH,
    MAP_MERGEPATH,
    MAP_ROWGROUP,
    MAP_SEGSCAN,
    SCHED_WIDE,
    CTX_NO_PROBE,
    CTX_VALIDATE,
    load as load_library,
)

load_library()

from .ops import (  # noqa: E402,F401
    Context,
    Hybrid,
    Transposed,
    attention,
    attention_backward,
    attention_qk_backward,
    attention_pipeline,
    attention_qk,
    candidates,
    default_context,
    default_schedule,
    degree_histogram,
    gather_values,
    inverse_permutation,
    permutation_plan,
    permute_values,
    PermutationPlan,
    hybrid_format,
    hybrid_parts,
    hybrid_plan,
    hybrid_problem,
    hybrid_sddmm,
    hybrid_select,
    hybrid_spmm,
    hybrid_values,
    make_problem,
    merge_path_partition,
    mha_attention,
    Plan,
    plan,
    plan_sddmm,
    plan_spmm,
    row_softmax,
    row_softmax_backward,
    sddmm,
    sddmm_backward,
    select,
    signature,
    spmm,
    spmm_sddmm,
    spmm_backward,
    spmm_transposed,
    spmm_noalloc,
    transpose,
    workspace_size,
)
