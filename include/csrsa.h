/*
 * csrsa.h - C ABI of an MI355X (gfx950) library for CSR sparse aggregation:
 * SpMM, SDDMM and softmax attention over a CSR pattern, with an input-aware
 * schedule selector and a persistent schedule cache.
 *
 * The operations are those of "AutoSAGE: Input-Aware CUDA Scheduling for
 * Sparse GNN Aggregation (SpMM/SDDMM) and CSR Attention" (Abstract): CSR SpMM,
 * CSR SDDMM, and their composition into a CSR attention pipeline
 * SDDMM -> row-softmax -> SpMM; a scheduler picks tiling and mapping per input
 * from a cheap estimate refined by on-device micro-probes, falls back to a
 * safe default, and keeps its choices in a persistent cache so that runs
 * replay deterministically.  The argument order and the edge-case rules of
 * the attention call follow the fused sparse attention-value aggregation task
 * on the POPCORNBENCH trace page (task statement; its host wrapper and final
 * kernel): row_ptr, col_idx, edge_scores, node_value; rows are destination
 * nodes, col_idx holds the source node of each incoming edge, the number of
 * nodes is len(row_ptr) - 1, the feature width is node_value's second
 * dimension, and a node without incoming edges gets a zero output row.
 *
 * Conventions for every call below
 *  - Pointers named row_ptr, col_idx, vals, X, U, V, Q, K, edge_scores,
 *    node_value, out, Y and workspace are DEVICE pointers (memory of the GPU
 *    the context was created on).  Every other pointer is a host pointer.
 *  - row_ptr: int32 [n_rows + 1], row_ptr[0] = 0, non-decreasing,
 *    row_ptr[n_rows] = nnz.  col_idx: int32 [nnz], each in [0, n_cols).
 *    Columns need not be sorted or unique; every stored entry counts once
 *    (duplicates add in SpMM and are separate terms of a row's softmax).
 *    The library never writes row_ptr or col_idx (they pass through bit-exact).
 *  - Dense matrices are row-major with a leading dimension (elements between
 *    consecutive rows) >= their width and < 2^30.  Index arithmetic is
 *    64-bit, so a dense operand may exceed 2^31 elements; nnz must be < 2^31.
 *  - Outputs are fully overwritten (including zero rows for rows without
 *    entries); no pre-zeroing is needed.  Inputs are never modified.
 *  - The caller owns all memory.  The library allocates no device memory on
 *    the call path; temporary storage comes from the caller's workspace,
 *    sized with csr_workspace_size().  The auto-select path also uses a small
 *    pinned host buffer owned by the context.
 *  - stream is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously.  Only the auto-select path (sched == NULL), validation
 *    (CSR_CTX_VALIDATE) and the calls marked "synchronous" wait on the
 *    stream; otherwise a call only enqueues kernels (no memset, no
 *    allocation), so it may be captured into a HIP graph.
 *  - Every call returns a csr_status (0 = CSR_OK).  No C++ exception or abort
 *    crosses the ABI.  On error nothing has been written to the outputs
 *    unless stated; csr_last_error() gives a message.
 *  - Calls on one context are serialised by an internal mutex, argument
 *    checks and error messages included, so a context may be shared by
 *    threads; csr_last_error() then gives the message of the last failed
 *    call from any thread, valid until the next call on the context.
 */
#ifndef CSRSA_H
#define CSRSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSRSA_ABI_VERSION 2
#define CSR_SCHEDULE_VERSION 1

typedef struct csr_context_s* csr_context_t;

enum csr_status {
    CSR_OK = 0,
    CSR_ERR_NULL = -1,           /* a required pointer is NULL */
    CSR_ERR_SHAPE = -2,          /* a size or leading dimension is invalid or unsupported */
    CSR_ERR_DTYPE = -3,          /* unsupported element type */
    CSR_ERR_ALIGN = -4,          /* misaligned pointer or leading dimension */
    CSR_ERR_WORKSPACE = -5,      /* workspace missing or too small */
    CSR_ERR_INVALID_CSR = -6,    /* CSR validation failed (context flag CSR_CTX_VALIDATE) */
    CSR_ERR_SCHEDULE = -7,       /* schedule invalid for this problem */
    CSR_ERR_NO_CACHE_ENTRY = -8, /* CSR_SELECT_REPLAY_ONLY and no cached schedule */
    CSR_ERR_CACHE_IO = -9,       /* cache file could not be read or written */
    CSR_ERR_HIP = -10,           /* a HIP runtime call failed */
    CSR_ERR_DEVICE = -11,        /* no usable gfx950 device */
    CSR_ERR_INTERNAL = -12
};

enum csr_op {
    CSR_OP_SPMM = 1,      /* Y = A X */
    CSR_OP_SDDMM = 2,     /* out_e = <U[row_e], V[col_e]> */
    CSR_OP_ATTENTION = 3, /* scores given: out = softmax_row(scale * S) V */
    CSR_OP_MHA = 4,       /* multi-head, scores = scale * <Q_i, K_j> per head */
    CSR_OP_ROW_SOFTMAX = 5, /* p_e = softmax over the row's entries of scale * s */
    CSR_OP_SOFTMAX_BWD = 6, /* ds_e = scale * p_e * (g_e - sum over the row of p g) */
    CSR_OP_ATTENTION_QK = 7, /* one head, scores = scale * <Q_i, K_j> formed in the same pass */
    CSR_OP_SPMM_SDDMM = 8   /* Y = A X and z_e = <U[row_e], X[col_e]> from one gather of X */
};

/* Element types of the dense operands.  bf16 operands are raw bfloat16 bit
 * patterns (uint16), widened exactly to fp32 on load; every op accumulates
 * and writes fp32.  bf16 operands of the lane-group ops (SpMM, SDDMM,
 * attention) need an even width, even leading dimensions and 4-byte aligned
 * rows (lane accesses of 2, 4 or 8 values). */
enum csr_dtype { CSR_DTYPE_F32 = 0, CSR_DTYPE_BF16 = 1 };

/* Row mappings (the "mapping" half of a schedule). */
enum csr_mapping {
    CSR_MAP_ROWGROUP = 1,  /* a group of W lanes per row, lanes across the feature width */
    CSR_MAP_MERGEPATH = 2, /* nnz-balanced merge-path chunks per wavefront; col_idx and
                              edge values staged in LDS; split rows combined by a
                              deterministic fix-up pass */
    CSR_MAP_SEGSCAN = 3    /* small widths (SpMM, SDDMM): merge-path chunks staged in LDS,
                              lanes over consecutive entries, each lane gathering a whole
                              feature row; SpMM rows summed by a cross-lane segmented
                              scan.  group_lanes = 1, vec * passes covers the width,
                              passes <= 4, long_row = 0.  Row softmax: each lane owns a
                              run of chunk_items / 64 consecutive entries, rows crossing
                              lanes completed by one segmented scan per chunk
                              (group_lanes 1, long_row 0, chunk_items 256, 512, 1024) */
};

/* Schedule flags. */
enum csr_schedule_flags {
    /* 16-byte lane accesses over rows that are only 4-byte aligned or whose
     * width is not a multiple of 4: vec 4, 64 lanes per row, passes = the
     * fewest supported counts covering width / 256; the lane whose 4 floats
     * would pass the width reads the 4 ending at it (so every access stays
     * inside its row, the last row of X included) and uses the top ones.
     * SpMM with the row-group mapping only, width >= 4. */
    CSR_SCHED_WIDE = 1
};

/* Context flags. */
enum csr_ctx_flags {
    CSR_CTX_VALIDATE = 1u,   /* check row_ptr / col_idx on every call (one extra pass) */
    CSR_CTX_NO_PROBE = 2u    /* never run micro-probes: cost model only */
};

/* Selection modes for csr_select(). */
enum csr_select_mode {
    CSR_SELECT_AUTO = 0,        /* cache hit -> replay; miss -> estimate + probes, then store */
    CSR_SELECT_REPLAY_ONLY = 1, /* cache only; CSR_ERR_NO_CACHE_ENTRY on a miss */
    CSR_SELECT_FORCE_PROBE = 2, /* ignore the cache, probe, store (replaces the entry) */
    CSR_SELECT_ESTIMATE = 3     /* cost model only, nothing stored */
};

/*
 * A schedule: plain data, 64 bytes, safe to copy, store and compare with
 * memcmp.  Obtain one from csr_select() or csr_default_schedule(); passing
 * a schedule back replays it without any host-side work beyond argument
 * checks.  Fields are validated against the problem on every call
 * (CSR_ERR_SCHEDULE if they do not fit).
 */
typedef struct csr_schedule_s {
    int32_t version;     /* CSR_SCHEDULE_VERSION */
    int32_t op;          /* enum csr_op */
    int32_t mapping;     /* enum csr_mapping */
    int32_t vec;         /* elements per lane access: 1, 2, 4 (fp32 operands); 2, 4, 8 (bf16) */
    int32_t group_lanes; /* W: lanes per row group, power of two in [1, 64] */
    int32_t passes;      /* feature passes per lane (width = W * vec * passes, rounded) */
    int32_t chunk_items; /* merge-path: rows + entries per wavefront chunk (256, 512, 1024) */
    int32_t long_row;    /* merge-path: a row segment this long is shared by the whole wave */
    int32_t flags;       /* enum csr_schedule_flags (0 = none) */
    int32_t reserved[7]; /* 0 */
} csr_schedule_t;

/*
 * A problem description: the same fields as the operation calls, used by
 * csr_select() and csr_workspace_size().  Unused pointers may be NULL for
 * csr_workspace_size().
 *   op = CSR_OP_SPMM:      a = vals (fp32 [nnz], NULL = all ones), b = X (dtype), width = F,
 *                          ld_b = ldx, out = Y, ld_out = ldy
 *   op = CSR_OP_SDDMM:     a = U [n_rows, K], ld_a = ldu, b = V [n_cols, K], ld_b = ldv
 *                          (both of dtype), width = K, out = fp32 [nnz]
 *   op = CSR_OP_ATTENTION: a = edge_scores fp32 [nnz], b = node_value [n_cols, F],
 *                          ld_b, width = F, out [n_rows, F], ld_out, scale
 *   op = CSR_OP_MHA:       a = Q, b = K, c = V (bf16 [n, heads, head_dim]), heads,
 *                          head_dim, width = heads * head_dim, out fp32 [n_rows, width],
 *                          scale
 *   op = CSR_OP_ROW_SOFTMAX: a = scores fp32 [nnz], out = probabilities fp32 [nnz],
 *                          width = 1, scale (n_cols is not used)
 *   op = CSR_OP_ATTENTION_QK: one head of an attention from queries and keys:
 *                          a = Q [n_rows, ld_a], b = K [n_cols, ld_b], c = V [n_cols, ld_c]
 *                          (all of dtype), width = head_dim (<= 1024), out fp32
 *                          [n_rows, ld_out], scale
 *   op = CSR_OP_SPMM_SDDMM: a = vals (fp32 [nnz] or NULL = all ones), a_idx (optional),
 *                          b = X fp32 [n_cols, ld_b], c = U fp32 [n_rows, ld_c],
 *                          width = F, out = Y fp32 [n_rows, ld_out], out2 = z fp32,
 *                          out2_idx (optional)
 *   probs (attention ops, optional): the softmax probability of every entry,
 *   at probs[e * probs_stride] (stride 0 means 1); multi-head: [nnz, heads].
 */
typedef struct csr_problem_s {
    int32_t op;
    int32_t dtype;
    int64_t n_rows, n_cols, nnz;
    int64_t width;
    int32_t heads, head_dim;
    int64_t ld_a, ld_b, ld_out;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const void* a;
    const void* b;
    const void* c;
    void* out;
    float scale;
    int32_t pad_;
    void* workspace;
    size_t workspace_bytes;
    void* stream;
    int64_t ld_c;          /* CSR_OP_ATTENTION_QK: leading dimension of c */
    float* probs;          /* attention ops: per-entry probabilities out, or NULL */
    int64_t probs_stride;  /* floats between consecutive entries' probabilities (0: 1) */
    const int32_t* a_idx;  /* CSR_OP_SPMM, CSR_OP_SPMM_SDDMM: entry e's value is a[a_idx[e]] (NULL: a[e]) */
    float* out2;           /* CSR_OP_SPMM_SDDMM: the per-entry output z */
    const int32_t* out2_idx; /* CSR_OP_SPMM_SDDMM: z_e is written at out2[out2_idx[e]] (NULL: out2[e]) */
} csr_problem_t;

/* ---------------------------------------------------------------------------
 * Context
 * ------------------------------------------------------------------------- */

/* Creates a context on HIP device `device` (must be gfx950), or a host-only
 * context for device = -1 (cache and host-side calls only; operations return
 * CSR_ERR_DEVICE).  cache_path:
 * the persistent schedule cache, an append-only text log (NULL = in-memory
 * only).  An existing log is loaded; malformed or foreign-version lines are
 * skipped.  flags: enum csr_ctx_flags.  The context owns a 4 KiB pinned host
 * buffer and the in-memory cache. */
int csr_context_create(csr_context_t* ctx, int device, const char* cache_path, uint32_t flags);

/* Flushes the cache log and frees the context.  NULL is accepted. */
int csr_context_destroy(csr_context_t ctx);

/* Static message for a status code. */
const char* csr_status_string(int status);

/* Message of the last failed call on this context (valid until the next call). */
const char* csr_last_error(csr_context_t ctx);

/* ---------------------------------------------------------------------------
 * Operations
 *
 * sched: NULL selects a schedule automatically (degree histogram on the device,
 * a stream synchronisation to read it, cache lookup, and on a miss cost model
 * plus micro-probes that run the operation itself on the caller's operands);
 * otherwise the given schedule is replayed with no synchronisation.
 * workspace / ws_bytes: device scratch of at least csr_workspace_size() bytes
 * for this problem and schedule (for sched == NULL: the size reported for a
 * NULL schedule, which covers every candidate).  256-byte alignment required.
 * ------------------------------------------------------------------------- */

/* SpMM (AutoSAGE page, Abstract: CSR SpMM):
 *   Y[i, f] = sum over stored entries e of row i of vals[e] * X[col_idx[e], f]
 * vals: fp32 [nnz] or NULL (all ones).  X: [n_cols, ldx] of x_dtype
 * (CSR_DTYPE_F32, or CSR_DTYPE_BF16 bit patterns), F <= ldx.  Y: fp32
 * [n_rows, ldy], F <= ldy.  1 <= F <= 4096.  Accumulation is fp32 for both
 * dtypes.  CSR_ERR_DTYPE for another dtype; bf16 X with an odd width:
 * CSR_ERR_SHAPE; with odd ldx or rows not 4-byte aligned: CSR_ERR_ALIGN. */
int csr_spmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
             const int32_t* row_ptr, const int32_t* col_idx, const float* vals,
             const void* X, int32_t x_dtype, int64_t F, int64_t ldx, float* Y, int64_t ldy,
             const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream);

/* SpMM with the values read through an index (SparseTIR page, Abstract:
 * sparse operators of GNN training; the backward's dX = A^T dY):
 *   Y[i, f] = sum over stored entries e of row i of vals[val_idx[e]] * X[col_idx[e], f]
 * With the pattern and t_perm of csr_transpose this is the SpMM of A^T whose
 * values stay in A's order: no csr_gather_values pass, no copy of the values
 * in the transposed order.  vals: fp32, not NULL; val_idx: int32 [nnz], every
 * index in [0, nnz) (checked only with CSR_CTX_VALIDATE: CSR_ERR_INVALID_CSR;
 * an index out of range otherwise reads outside vals).  Other arguments,
 * rules and errors as for csr_spmm. */
int csr_spmm_perm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
                  const int32_t* row_ptr, const int32_t* col_idx, const float* vals, const int32_t* val_idx,
                  const void* X, int32_t x_dtype, int64_t F, int64_t ldx, float* Y, int64_t ldy,
                  const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream);

/* SpMM and SDDMM on one pattern sharing the gathered operand (AutoSAGE page,
 * Abstract: CSR SpMM and CSR SDDMM; SparseTIR page, Abstract: sparse
 * operators of GNN training):
 *   Y[i, f] = sum over stored entries e of row i of w_e * X[col_idx[e], f]
 *   z[t_e] = sum over f of U[i, f] * X[col_idx[e], f]   (e a stored entry of row i)
 * with w_e = vals[val_idx[e]] (val_idx given), vals[e], or 1 (vals NULL), and
 * t_e = z_idx[e] (z_idx given) or e.  Each gathered row X[col_idx[e], :] is
 * read once for both products.  On the pattern of A^T (csr_transpose) with
 * X = dOut, U = V, vals = P, val_idx = z_idx = t_perm, this gives in one pass
 * the two products of the backward of out = P V that read dOut: dV = P^T dOut
 * and dP = dOut V^T, the latter at A's entry positions.
 * X: fp32 [n_cols, ldx]; U: fp32 [n_rows, ldu]; Y: fp32 [n_rows, ldy]
 * (F <= ldx, ldu, ldy; 1 <= F <= 4096); z: fp32 [nnz].  val_idx, z_idx:
 * int32 [nnz], every index
 * in [0, nnz) (checked only with CSR_CTX_VALIDATE: CSR_ERR_INVALID_CSR; an
 * index out of range otherwise reads or writes outside vals or z); the
 * entries of z_idx must be distinct (a permutation, as t_perm is): two
 * entries with one slot leave either value in it.  Operands are fp32 (the
 * call has no dtype argument); schedules take the row-group or merge-path
 * mapping and no flags.  Other rules and errors as for csr_spmm. */
int csr_spmm_sddmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
                   const int32_t* row_ptr, const int32_t* col_idx, const float* vals,
                   const int32_t* val_idx, const float* X, int64_t F, int64_t ldx,
                   const float* U, int64_t ldu, float* Y, int64_t ldy, float* z,
                   const int32_t* z_idx, const csr_schedule_t* sched, void* workspace,
                   size_t ws_bytes, void* stream);

/* Scratch capacity (bytes per GPU) of csr_spmm_noalloc. */
#define CSR_NOALLOC_SCRATCH_BYTES (32u << 20)

/* csr_spmm for callers that cannot allocate memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, result and errors as csr_spmm with an explicit schedule, but
 * without a workspace: the kernels' scratch (merge-path coordinates and
 * split-row pieces) lives in a device array of CSR_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends.  Nothing
 * is allocated and nothing synchronised (unless the context validates).
 * sched must not be NULL (select it once beforehand: CSR_ERR_NULL);
 * problems whose schedule needs more scratch than the array holds
 * (csr_workspace_size > CSR_NOALLOC_SCRATCH_BYTES) are refused with
 * CSR_ERR_WORKSPACE before anything is enqueued; CSR_ERR_HIP if the array's
 * address could not be obtained for the context's device.  Every call on a
 * GPU uses that GPU's one array, whatever the context or stream: calls whose
 * kernels overlap in time on one GPU race and must be ordered by the caller
 * (one stream, or events).  No scratch content has to start at zero. */
int csr_spmm_noalloc(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
                     const int32_t* row_ptr, const int32_t* col_idx, const float* vals,
                     const void* X, int32_t x_dtype, int64_t F, int64_t ldx, float* Y, int64_t ldy,
                     const csr_schedule_t* sched, void* stream);

/* SDDMM (AutoSAGE page, Abstract: CSR SDDMM):
 *   out[e] = sum over k < K of U[i, k] * V[col_idx[e], k] for every stored
 *   entry e of row i, in CSR order.
 * U: [n_rows, ldu], V: [n_cols, ldv], both of dtype (CSR_DTYPE_F32 or
 * CSR_DTYPE_BF16); out: fp32 [nnz], fp32 accumulation.  1 <= K <= 4096.
 * bf16 rules and errors as for csr_spmm. */
int csr_sddmm(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
              const int32_t* row_ptr, const int32_t* col_idx,
              const void* U, int64_t ldu, const void* V, int64_t ldv, int32_t dtype, int64_t K,
              float* out, const csr_schedule_t* sched, void* workspace, size_t ws_bytes,
              void* stream);

/* Fused CSR attention (AutoSAGE page, Abstract: the SDDMM -> row-softmax ->
 * SpMM pipeline; POPCORNBENCH trace page, task statement: argument order
 * row_ptr, col_idx, edge_scores, node_value).  For each row i with entries
 * E_i, head h, the scores t_e, p_e = exp(t_e - max t) / sum over E_i of
 * exp(t - max t), out[i, h, :] = sum over e in E_i of p_e * V[col_idx[e], h, :];
 * out[i, h, :] = 0 when E_i is empty.
 *   edge_scores != NULL, or Q and K both NULL (scores given): Q and K are
 *     not read, t_e = scale * edge_scores[h * nnz + e] (fp32 [heads, nnz],
 *     head-major: each head's scores contiguous, in entry order; NULL only
 *     when nnz = 0).  Several heads run as one-head problems on column
 *     views of V and out (schedule op CSR_OP_ATTENTION, shared by the
 *     heads).
 *   edge_scores == NULL and Q, K given (scores from queries and keys, one
 *     pass): t_e =
 *     scale * sum over d of Q[i, h, d] * K[col_idx[e], h, d]; Q: [n_rows,
 *     heads * head_dim] and K: [n_cols, heads * head_dim], rows contiguous.
 *     bf16 with head_dim a power of two in [8, 512], heads * head_dim <= 512,
 *     ldv = ldo = heads * head_dim and 16-byte aligned operands runs the
 *     multi-head kernel (schedule op CSR_OP_MHA); otherwise each head runs
 *     as one CSR_OP_ATTENTION_QK problem (head_dim <= 1024; schedule op
 *     CSR_OP_ATTENTION_QK, shared by the heads).
 * V = node_value: [n_cols, ldv] of dtype (CSR_DTYPE_F32, or CSR_DTYPE_BF16
 * bit patterns; Q and K of the same dtype), ldv >= heads * head_dim.  out:
 * fp32 [n_rows, ldo].  probs_out: NULL, or fp32 [nnz * heads], entry-major
 * (p of entry e, head h at probs_out[e * heads + h]).  scale: finite (1.0 =
 * no scaling).  Accumulation is fp32.  CSR_ERR_SHAPE for heads or head_dim
 * below 1 or ldv / ldo below heads * head_dim; other errors as for
 * csr_spmm. */
int csr_attention(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
                  const int32_t* row_ptr, const int32_t* col_idx, const float* edge_scores,
                  const void* Q, const void* K, const void* node_value, int32_t dtype,
                  int32_t heads, int64_t head_dim, int64_t ldv, float scale,
                  float* out, int64_t ldo, float* probs_out, const csr_schedule_t* sched,
                  void* workspace, size_t ws_bytes, void* stream);

/* Multi-head fused CSR attention, SDDMM -> row-softmax -> SpMM in one pass
 * (AutoSAGE page, Abstract: CSR attention pipeline), bf16 inputs, fp32
 * accumulation and output.  For each head h and row i:
 *   t_e = scale * sum over d of Q[i, h, d] * K[col_idx[e], h, d],
 *   p_e = softmax over the row's entries of t,
 *   out[i, h, d] = sum over e of p_e * V[col_idx[e], h, d]; zero for empty rows.
 * Q: bf16 [n_rows, heads, head_dim]; K, V: bf16 [n_cols, heads, head_dim]
 * (raw bfloat16 bit patterns, contiguous); out: fp32 [n_rows, heads, head_dim].
 * head_dim in {8, 16, 32, 64, 128, 256, 512}, heads * head_dim <= 512,
 * 16-byte aligned pointers.  probs_out: NULL, or fp32 [nnz, heads] (the
 * probability of every entry per head). */
int csr_mha_attention(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz,
                      const int32_t* row_ptr, const int32_t* col_idx,
                      const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                      int32_t heads, int32_t head_dim, float scale, float* out, float* probs_out,
                      const csr_schedule_t* sched, void* workspace, size_t ws_bytes,
                      void* stream);

/* CSR row softmax, the middle stage of the unfused pipeline SDDMM ->
 * row-softmax -> SpMM (AutoSAGE page, Abstract): for every stored entry e of
 * row i, probs[e] = exp(scale * scores[e] - m_i) / sum over the row's entries
 * of exp(scale * scores - m_i), m_i the row maximum of scale * scores.
 * scores, probs: fp32 [nnz] (may alias for an in-place update; an in-place
 * call with sched == NULL then picks its schedule by the cost model alone,
 * since a micro-probe would overwrite its own input).  Rows without entries
 * have nothing to write.  Schedules (vec 1, passes 1): the merge-path mapping
 * with group_lanes = lanes per short row and chunk_items 256 or 512, or the
 * segmented-scan mapping (lane-owned entry runs) with group_lanes 1, long_row 0
 * and chunk_items 256, 512 or 1024. */
int csr_row_softmax(csr_context_t ctx, int64_t n_rows, int64_t nnz, const int32_t* row_ptr,
                    const float* scores, float scale, float* probs, const csr_schedule_t* sched,
                    void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Backward operations (the gradients of the three products, for training the
 * GNN layers the AutoSAGE page's SpMM / SDDMM serve).  With Y = A X:
 * dX = A^T dY (csr_transpose + csr_gather_values + csr_spmm) and
 * d(edge values) = SDDMM(dY, X).  With out_e = <U_i, V_j>: dU = A_g V and
 * dV = A_g^T U.  For the attention, dV = P^T dOut, dP = SDDMM(dOut, V) and
 * d(scores) = csr_row_softmax_backward(P, dP).
 * ------------------------------------------------------------------------- */

/* Softmax backward over each row's stored entries: with p the row softmax of
 * scale * s and g = dL/dp, dL/ds_e = scale * p_e * (g_e - sum over the row of
 * p * g).  probs, grad_probs, grad_scores: fp32 [nnz] (grad_scores may alias
 * either input for an in-place update; an in-place call with sched == NULL
 * picks its schedule by the cost model alone).  Rows without entries have
 * nothing to write.  Schedules: the segmented-scan mapping (lane-owned entry
 * runs), vec 1, passes 1, group_lanes 1, long_row 0, chunk_items 256 or 512.
 * Errors as for csr_row_softmax. */
int csr_row_softmax_backward(csr_context_t ctx, int64_t n_rows, int64_t nnz, const int32_t* row_ptr,
                             const float* probs, const float* grad_probs, float scale, float* grad_scores,
                             const csr_schedule_t* sched, void* workspace, size_t ws_bytes, void* stream);


/* Device workspace (bytes) that csr_transpose needs for these sizes.
 * Returns CSR_ERR_SHAPE for negative sizes or sizes beyond int32 indices,
 * CSR_ERR_DEVICE on a host-only context. */
int csr_transpose_workspace_size(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, size_t* bytes);

/* The CSR pattern of A^T (A in CSC form): t_row_ptr int32 [n_cols + 1],
 * t_col_idx int32 [nnz] (the original row of each entry), t_perm int32 [nnz]
 * (the original entry index of each transposed entry, so that a value array v
 * of A becomes v[t_perm[k]] for A^T; see csr_gather_values).  The entries of
 * each column keep their original order (a stable sort by column): the result
 * is deterministic.  All arrays are caller-allocated device memory; the inputs
 * are not modified; workspace of csr_transpose_workspace_size bytes.  col_idx
 * must lie in [0, n_cols) (checked only with CSR_CTX_VALIDATE:
 * CSR_ERR_INVALID_CSR).  CSR_ERR_WORKSPACE when ws_bytes is too small. */
int csr_transpose(csr_context_t ctx, int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t* row_ptr,
                  const int32_t* col_idx, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm,
                  void* workspace, size_t ws_bytes, void* stream);

/* dst[k] = src[perm[k]] for k < n (fp32, src and dst of n values; dst must
 * not alias src; an index outside [0, n) gives 0): moves per-entry values
 * (edge values, probabilities, gradients) into the order of a transposed
 * pattern. */
int csr_gather_values(csr_context_t ctx, int64_t n, const int32_t* perm, const float* src, float* dst, void* stream);

/* inv[perm[k]] = k for k < n: the inverse of a permutation of [0, n) (for a
 * transposed pattern's t_perm: the position in A^T of each entry of A).  An
 * index of perm outside [0, n) is skipped (nothing is written for it); perm
 * must be a permutation for inv to be complete (not checked).  inv must not
 * alias perm (CSR_ERR_SHAPE when they are the same array).  CSR_ERR_SHAPE
 * for n < 0 or n >= 2^31. */
int csr_inverse_permutation(csr_context_t ctx, int64_t n, const int32_t* perm, int32_t* inv, void* stream);

/* A permutation of per-entry values in two passes: dst[e] = src[q[e]] for a
 * permutation q of [0, n) (q = t_perm moves values of A into A^T's order,
 * its inverse moves them back).  A direct gather reads a 4-byte value from a
 * random 128-byte line per entry; the plan groups the outputs by the window
 * of 2^window_log2 source values they read, so that the first pass reads one
 * window at a time (from the L2 of the XCD that holds it) and the second
 * reads the groups in contiguous runs.  The plan is two caller-allocated
 * int32 [n] device arrays q1 and pos (q1[j] = q[order[j]], pos[order[j]] = j
 * for the outputs in window order), built once per permutation by
 * csr_permutation_plan with workspace of csr_permutation_plan_workspace_size
 * bytes; q must be a permutation (not checked; an index outside [0, n)
 * makes the plan's results unspecified, never an access outside the
 * arrays).  window_log2 in [8, 30]; CSR_ERR_SHAPE otherwise or for n < 0 or
 * n >= 2^31.  csr_permute_values applies a plan: tmp[j] = src[q1[j]], then
 * dst[e] = tmp[pos[e]] (fp32; tmp [n] is caller scratch; src, tmp and dst
 * must not alias: CSR_ERR_SHAPE when two are the same array). */
int csr_permutation_plan_workspace_size(csr_context_t ctx, int64_t n, size_t* bytes);
int csr_permutation_plan(csr_context_t ctx, int64_t n, const int32_t* q, int32_t window_log2, int32_t* q1,
                         int32_t* pos, void* workspace, size_t ws_bytes, void* stream);
int csr_permute_values(csr_context_t ctx, int64_t n, const int32_t* q1, const int32_t* pos, const float* src,
                       float* tmp, float* dst, void* stream);

/* ---------------------------------------------------------------------------
 * Column-part segment format (a composed, "hybrid" format)
 *
 * The SparseTIR page (abstract) holds that no single sparse format gets full
 * hardware efficiency on every input and that formats should be composed.
 * This format composes a partition of the columns with a compaction of the
 * rows: the columns are cut into P equal parts (column c lies in part
 * c / part_cols, part_cols = ceil(n_cols / P)); a segment is the run of one
 * row's entries whose columns lie in one part (the entries keep their
 * original order); the segments are ordered by (part, row) and only non-empty
 * segments are stored.  A row with fewer than whole_below entries is not
 * split: its entries form one segment in an extra part P, after all the
 * column parts (a short row would otherwise make about one segment per
 * entry).  The segments form a plain CSR pattern (seg_ptr over
 * the reordered entries, n_seg rows), so every mapping of the plain products
 * runs on it; blocks reach the parts in order, so at any time the gathered
 * rows of the dense operand come from about one 1/P slice of it, a slice that
 * the caches hold.  A product over the format equals the plain product up to
 * the order of the additions (a row's segments are summed in part order).
 * ------------------------------------------------------------------------- */
typedef struct csr_hybrid_s {
    int64_t n_rows, n_cols, nnz; /* the pattern's shape (set by the caller) */
    int32_t parts;               /* P: a power of two from 1 to 256 (set by the caller) */
    int32_t part_cols;           /* ceil(n_cols / P) (written by csr_hybrid_build) */
    int32_t whole_below;         /* rows with fewer entries are kept whole: one segment in
                                    part P, after all column parts; 0 = split every row
                                    (set by the caller) */
    int32_t reserved_;           /* must be 0 */
    int64_t seg_cap;             /* capacity of the segment arrays, >= csr_hybrid_capacity (set by the caller) */
    int64_t n_seg;               /* number of segments (written by csr_hybrid_build) */
    int32_t* perm;               /* [nnz] original entry index of each format entry */
    int32_t* col_idx;            /* [nnz] column of each format entry */
    int32_t* seg_ptr;            /* [seg_cap + 1] first format entry of each segment; seg_ptr[n_seg] = nnz */
    int32_t* seg_row;            /* [seg_cap] row of each segment */
    int32_t* row_seg_ptr;        /* [n_rows + 1] each row's slots in row_seg */
    int32_t* row_seg;            /* [seg_cap] each row's segments, in part order */
} csr_hybrid_t;

/* The format's plan for problem p (op CSR_OP_SPMM or CSR_OP_SDDMM; shape
 * fields only) with degree histogram (int64 [67], or NULL): the column parts
 * (1 when the plain CSR path is expected to be faster) and the whole-row
 * threshold (whole_below may be NULL).  A cost model measured on MI355X:
 * the gathers of the split rows cost least while one part holds about 4 MiB
 * of the gathered matrix (one XCD's L2), the rows kept whole gather from all
 * of it, and every segment's partial row is written and read once; the
 * segment count is expected from the histogram.  Parts 4 ... 256 and
 * power-of-two thresholds are scored; the format is proposed when it is
 * estimated at least 5 % faster.  SDDMM: rows of at most 16 floats, about
 * 4 MiB per part, every row split.  Host-only. */
int csr_hybrid_plan(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, int32_t* parts,
                    int32_t* whole_below);

/* The parts of csr_hybrid_plan.  Host-only. */
int csr_hybrid_parts(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram, int32_t* parts);

/* Upper bound of the segment count, min(nnz, n_rows * parts): the capacity
 * the segment arrays need.  Host-only; CSR_ERR_SHAPE for bad sizes or
 * parts. */
int csr_hybrid_capacity(int64_t n_rows, int64_t nnz, int32_t parts, int64_t* seg_cap);

/* Device workspace (bytes) that csr_hybrid_build needs for these sizes. */
int csr_hybrid_build_workspace_size(csr_context_t ctx, int64_t n_rows, int64_t nnz, int32_t parts, size_t* bytes);

/* Builds the format of the CSR pattern (row_ptr, col_idx) into the
 * caller-allocated device arrays of *h (sizes and parts set by the caller;
 * part_cols and n_seg are written).  Deterministic (stable sorts, no
 * order-dependent atomics).  Synchronous: it reads the segment count back.
 * col_idx must lie in [0, n_cols) (checked only with CSR_CTX_VALIDATE:
 * CSR_ERR_INVALID_CSR).  CSR_ERR_WORKSPACE when ws_bytes or h->seg_cap is too
 * small. */
int csr_hybrid_build(csr_context_t ctx, const int32_t* row_ptr, const int32_t* col_idx, csr_hybrid_t* h,
                     void* workspace, size_t ws_bytes, void* stream);

/* Device workspace (bytes) of csr_hybrid_spmm (op CSR_OP_SPMM: includes the
 * segments' partial rows, n_seg * width floats) or csr_hybrid_sddmm (op
 * CSR_OP_SDDMM) at this width and dtype, for schedule sched (NULL: any the
 * selector may pick).  h must be built. */
int csr_hybrid_workspace_size(csr_context_t ctx, const csr_hybrid_t* h, int32_t op, int64_t width, int32_t dtype,
                              const csr_schedule_t* sched, size_t* bytes);

/* Y = A X over a built format: each segment's product into its partial row
 * (a CSR SpMM of the n_seg-row segment pattern, any mapping), then
 * Y[r] = the sum of row r's partial rows in part order (+0 for a row without
 * entries).  vals: [nnz] edge values in FORMAT order (csr_gather_values with
 * h->perm moves them there), or NULL for all ones.  X, x_dtype, F, ldx, Y,
 * ldy as for csr_spmm.  sched: a schedule of op CSR_OP_SPMM for the segment
 * pattern (NULL: selected and cached as for csr_spmm, keyed by the segment
 * pattern's shape and degree histogram). */
int csr_hybrid_spmm(csr_context_t ctx, const csr_hybrid_t* h, const float* vals, const void* X, int32_t x_dtype,
                    int64_t F, int64_t ldx, float* Y, int64_t ldy, const csr_schedule_t* sched, void* workspace,
                    size_t ws_bytes, void* stream);

/* out[e] = dot(U[row(e)], V[col(e)]) over a built format, written in the
 * ORIGINAL entry order (the kernels read U through seg_row and write through
 * perm).  U, ldu, V, ldv, dtype, K, out as for csr_sddmm; sched: a schedule
 * of op CSR_OP_SDDMM for the segment pattern (NULL: selected). */
int csr_hybrid_sddmm(csr_context_t ctx, const csr_hybrid_t* h, const void* U, int64_t ldu, const void* V,
                     int64_t ldv, int32_t dtype, int64_t K, float* out, const csr_schedule_t* sched, void* workspace,
                     size_t ws_bytes, void* stream);

/* Selects (and caches) the schedule of the segment product of a call over a
 * built format, as csr_select does for a plain call.  call describes the
 * call's operands only: op (CSR_OP_SPMM or CSR_OP_SDDMM), dtype, width, a / ld_a
 * (SpMM: the format-order values or NULL; SDDMM: U), b / ld_b (X or V), out
 * (SDDMM: the [nnz] output, written by the probes; SpMM: unused, the probes
 * write the partial rows into the workspace), workspace (of
 * csr_hybrid_workspace_size bytes), workspace_bytes and stream; its pattern
 * fields are ignored.  Modes and the signature as for csr_select. */
int csr_hybrid_select(csr_context_t ctx, const csr_hybrid_t* h, const csr_problem_t* call, uint32_t mode,
                      csr_schedule_t* out, uint64_t* signature);

/* ---------------------------------------------------------------------------
 * Planned products: one CSR matrix prepared for one SpMM or SDDMM (AutoSAGE
 * page, Abstract: tiling and mapping chosen per input by an estimate refined
 * with on-device micro-probes, kept in a persistent cache for deterministic
 * replay; SparseTIR page, Abstract: composed formats searched over).  The
 * library chooses the layout and the schedule together: the plain CSR
 * pattern, or the column-part segment format above at several part counts
 * and whole-row thresholds, each with the schedules of its product; the
 * joint choice is cached under the input's signature (a log line of its
 * own) and replayed on later plans of the same input.  The plan's arrays
 * (the format, the values in format order) live in caller memory sized by
 * csr_plan_size.
 * ------------------------------------------------------------------------- */
#define CSR_PLAN_VERSION 2

/* Degree classes (SparseTIR page, Abstract: composable formats; rows
 * bucketed by degree, the short ones packed ELL-style): the rows with 1 to
 * short_below - 1 entries are grouped by class c = 1 .. n_classes (degrees
 * [2^(c-1), 2^c)), each class padded to 2^c - 1 slots per row and stored
 * slot-major (slot j of the class's row i at class_base + j * rows_in_class
 * + i), so that a row per lane group reads its slots with the loads of the
 * neighbouring rows; the other rows (empty or long) form a CSR of their own
 * on the same row numbering, in which the packed rows are empty.  SpMM only.
 * Built by csr_plan_create into the plan memory. */
#define CSR_BUCKET_MAX_CLASSES 6

typedef struct csr_bucket_s {
    int32_t short_below;      /* 2, 4, ..., 64: rows with fewer entries (and at least one) are packed */
    int32_t n_classes;        /* log2(short_below) */
    int64_t n_short;          /* packed rows */
    int64_t n_slots;          /* packed slots, entries and padding */
    int64_t nnz_long;         /* entries of the other rows */
    int64_t class_rows[CSR_BUCKET_MAX_CLASSES]; /* rows of classes 1 .. n_classes */
    int32_t* rows;            /* [n_rows]: the packed rows, class by class, each class in row order */
    int32_t* slot_col;        /* [n_slots] column of each slot, -1 for padding (after a row's entries) */
    int32_t* slot_pos;        /* [n_slots] the entry behind each slot, -1 for padding */
    float* slot_val;          /* [n_slots] its value (0 for padding) */
    int32_t* long_row_ptr;    /* [n_rows + 1] the other rows' CSR */
    int32_t* long_col;        /* [nnz_long] */
    int32_t* long_pos;        /* [nnz_long] the entry behind each long entry */
    float* long_val;          /* [nnz_long] */
} csr_bucket_t;

typedef struct csr_plan_s {
    int32_t version;          /* CSR_PLAN_VERSION */
    int32_t op;               /* CSR_OP_SPMM or CSR_OP_SDDMM */
    int32_t dtype;            /* element type of the dense operands */
    int32_t parts;            /* 1: the plain pattern; 0: degree classes (bkt); otherwise the
                                 column-part format's parts (fmt) */
    int32_t whole_below;      /* the format's whole-row threshold; with parts 0, bkt.short_below */
    int32_t reserved_;
    int64_t n_rows, n_cols, nnz, width;
    uint64_t signature;       /* the cache key of the choice */
    csr_schedule_t sched;     /* the product's schedule (on the segment pattern when parts > 1, on
                                 the long rows' CSR when parts is 0) */
    csr_hybrid_t fmt;         /* the format (parts > 1), its arrays in the plan memory */
    csr_bucket_t bkt;         /* the degree classes (parts 0), their arrays in the plan memory */
    const int32_t* row_ptr;   /* the plain pattern: the caller's arrays, which must stay valid */
    const int32_t* col_idx;
    float* vals;              /* SpMM: the values the product reads (the caller's array on the
                                 plain pattern, the plan's format-order copy otherwise; NULL: 1) */
    size_t workspace_bytes;   /* workspace of csr_plan_spmm / csr_plan_sddmm */
    double probe_ms;          /* probed time of the choice (0 when replayed or estimated) */
} csr_plan_t;

/* Sizes for planning problem p (op CSR_OP_SPMM or CSR_OP_SDDMM; shape,
 * dtype, leading dimensions, operand pointers for their alignment, row_ptr,
 * and a workspace of at least 1 KiB for the degree histogram): plan memory
 * and workspace that csr_plan_create needs for every layout it may probe
 * (the segment counts bounded from the degree histogram).  The workspace
 * also serves the planned calls.  Synchronous (reads the histogram). */
int csr_plan_size(csr_context_t ctx, const csr_problem_t* p, size_t* plan_bytes, size_t* workspace_bytes);

/* Plans problem p (every operand set, as for csr_select; SpMM: a = the
 * values in original order or NULL for ones, b = X; SDDMM: a = U, b = V;
 * out written by the probes) into *plan, with plan_mem (plan_bytes of
 * device memory, 256-byte aligned) holding the plan's arrays and
 * p->workspace of csr_plan_size's workspace bytes.  mode as for csr_select:
 * AUTO replays a cached choice or probes and caches one, REPLAY_ONLY
 * (CSR_ERR_NO_CACHE_ENTRY on a miss), FORCE_PROBE, ESTIMATE (the cost model
 * alone, nothing stored).  A layout whose every probe fails is never
 * chosen; if all fail, the plain pattern with its default schedule.  The
 * plan keeps pointers to row_ptr, col_idx and (plain SpMM) the values:
 * they must outlive it.  Synchronous. */
int csr_plan_create(csr_context_t ctx, const csr_problem_t* p, uint32_t mode, void* plan_mem, size_t plan_bytes,
                    csr_plan_t* plan);

/* Sizes for a plan of p in one given layout: parts 1 (the plain pattern),
 * 2 .. 256 (the column-part format, a power of two, whole_below >= 0 its
 * whole-row threshold) or 0 (SpMM: degree classes, whole_below the short
 * threshold, a power of two from 2 to 64).  As csr_plan_size otherwise;
 * CSR_ERR_SHAPE for a layout outside these rules. */
int csr_plan_layout_size(csr_context_t ctx, const csr_problem_t* p, int32_t parts, int32_t whole_below,
                         size_t* plan_bytes, size_t* workspace_bytes);

/* Plans p in the given layout (rules of csr_plan_layout_size) with schedule
 * sched for the product on that layout (the plain pattern, the segment
 * pattern of the format, or the long rows of the degree classes), or with
 * sched NULL the selector's choice for it (csr_select on that product, with
 * its cache).  For replaying a known choice and for measuring layouts one
 * by one; no plan choice is cached.  plan memory and workspace of
 * csr_plan_layout_size.  CSR_ERR_SCHEDULE when sched does not fit the
 * layout's product.  Synchronous. */
int csr_plan_build(csr_context_t ctx, const csr_problem_t* p, int32_t parts, int32_t whole_below,
                   const csr_schedule_t* sched, void* plan_mem, size_t plan_bytes, csr_plan_t* plan);

/* Y = A X with a plan of op CSR_OP_SPMM: X [n_cols, ldx] of the plan's dtype,
 * Y fp32 [n_rows, ldy], with the alignment and leading-dimension class the
 * plan was made for (CSR_ERR_SCHEDULE otherwise).  vals: NULL uses the
 * plan's values (those it was created with); otherwise this call's values
 * in original order, for this call only (over the format they are moved
 * into format order inside the workspace first).  No synchronisation; a
 * workspace of plan->workspace_bytes. */
int csr_plan_spmm(csr_context_t ctx, const csr_plan_t* plan, const float* vals, const void* X, int64_t ldx,
                  float* Y, int64_t ldy, void* workspace, size_t ws_bytes, void* stream);

/* out[e] = <U[row_e], V[col_e]> (original entry order) with a plan of op
 * CSR_OP_SDDMM; operands as for csr_sddmm, of the plan's dtype. */
int csr_plan_sddmm(csr_context_t ctx, const csr_plan_t* plan, const void* U, int64_t ldu, const void* V, int64_t ldv,
                   float* out, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Schedule selection and cache (AutoSAGE page, Abstract: input-aware choice
 * refined by on-device micro-probes, guarded fallback, persistent cache for
 * deterministic replay).
 * ------------------------------------------------------------------------- */

/* Selects a schedule for problem p (all operand pointers, workspace and stream
 * must be set unless mode == CSR_SELECT_REPLAY_ONLY or CSR_SELECT_ESTIMATE).
 * Probing runs the operation on p's operands and writes p->out.
 * signature (may be NULL) receives the 64-bit input signature: FNV-1a over
 * the problem shape, the degree histogram and the device identity.
 * Synchronous. */
int csr_select(csr_context_t ctx, const csr_problem_t* p, uint32_t mode,
               csr_schedule_t* out, uint64_t* signature);

/* The library's safe default schedule for p (the fallback when probing fails):
 * needs only the shape fields (and the operand pointers for their alignment).
 * Host-only; ctx may be NULL. */
int csr_default_schedule(csr_context_t ctx, const csr_problem_t* p, csr_schedule_t* out);

/* The candidate schedules the selector considers for p given its degree
 * histogram (int64 [67], or NULL), in the fixed order used for tie-breaking;
 * the first is csr_default_schedule().  Writes at most max entries to out and
 * the full count to *n.  Host-only; ctx may be NULL. */
int csr_candidates(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram,
                   csr_schedule_t* out, int32_t max, int32_t* n);

/* Workspace bytes needed for p under schedule sched (NULL = automatic
 * selection, covering every candidate).  Host-only; ctx may be NULL; needs
 * only the shape fields of p (and the operand pointers for their alignment). */
int csr_workspace_size(csr_context_t ctx, const csr_problem_t* p, const csr_schedule_t* sched,
                       size_t* bytes);

/* Appends to the log every in-memory entry that is not yet in it (entries
 * whose earlier append failed).  CSR_ERR_CACHE_IO if an append fails again. */
int csr_cache_flush(csr_context_t ctx);

/* Cache statistics (host-only; any pointer may be NULL): number of entries
 * (schedules and plans),
 * log lines skipped at load (malformed, truncated or of another schema
 * version), failed log appends. */
int csr_cache_info(csr_context_t ctx, int64_t* entries, int64_t* skipped_lines, int64_t* io_errors);

/* Looks up / stores the schedule cached for a signature (host-only).  A store
 * replaces the in-memory entry and appends one log line; on reload the last
 * valid line of a signature wins.  Store returns CSR_ERR_CACHE_IO when the
 * append fails (the entry is kept in memory). */
int csr_cache_lookup(csr_context_t ctx, uint64_t signature, csr_schedule_t* out);
int csr_cache_store(csr_context_t ctx, uint64_t signature, const csr_schedule_t* sched);

/* ---------------------------------------------------------------------------
 * Building blocks, exposed for testing and reuse
 * ------------------------------------------------------------------------- */

/* Degree histogram of a CSR pattern (the selector's input features).  Row i
 * has degree d = row_ptr[i+1] - row_ptr[i]; bucket 0 counts empty rows and
 * bucket b in 1..32 the rows with 2^(b-1) <= d < 2^b.
 * out_host: int64 [67] = counts[33], degree sums[33], max degree.
 * workspace: >= 1024 bytes.  Synchronous. */
int csr_degree_histogram(csr_context_t ctx, int64_t n_rows, const int32_t* row_ptr,
                         int64_t* out_host, void* workspace, size_t ws_bytes, void* stream);

/* Merge-path partition of rows + entries into chunks of items_per_chunk
 * items (items = row ends + stored entries, the end of a row following its
 * last entry).  coords: device int32 [2 * (n_chunks + 1)], (x, y) pairs =
 * (rows ended, entries consumed) before each chunk; the last pair is
 * (n_rows, nnz).  n_chunks = ceil((n_rows + nnz) / items_per_chunk), at least
 * 1.  Asynchronous. */
int csr_merge_path_partition(csr_context_t ctx, int64_t n_rows, int64_t nnz,
                             const int32_t* row_ptr, int32_t items_per_chunk,
                             int32_t* coords, void* stream);

/* Signature of problem p given its degree histogram (int64 [67] as returned
 * by csr_degree_histogram): FNV-1a 64 over the little-endian int64 sequence
 * 0x43535253, library version 1, op, dtype, n_rows, n_cols, nnz, width,
 * heads, head_dim (0, 0 for the fp32 ops), the widest vector access the
 * operands allow (1, 2, 4; 8 for multi-head), the device's CU count and
 * architecture number (950; both 0 when ctx is NULL or host-only), then the
 * 67 histogram values.  Host-only. */
int csr_signature(csr_context_t ctx, const csr_problem_t* p, const int64_t* histogram,
                  uint64_t* signature);

#ifdef __cplusplus
}
#endif

#endif /* CSRSA_H */
