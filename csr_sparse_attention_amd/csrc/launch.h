// Host-side launchers of the templated kernels (one translation unit per op).
#pragma once

#include <hip/hip_runtime.h>

#include "args.h"

namespace csrk {

// Feature passes per lane that have a kernel instantiation.
inline bool nv_supported(int nv)
{
    switch (nv) {
    case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 12: case 16: return true;
    default: return false;
    }
}
inline int nv_round_up(int nv)
{
    static const int s[] = {1, 2, 3, 4, 5, 6, 8, 12, 16};
    for (int v : s)
        if (v >= nv) return v;
    return -1;
}
inline bool chunk_supported(int d) { return d == 256 || d == 512 || d == 1024; }

// Entries in flight per lane group, from the registers one entry needs.
constexpr int unroll_for(int vec, int nv)
{
    return (vec * nv <= 2) ? 8 : (vec * nv <= 16) ? 4 : 2;
}

// Returns hipSuccess or the launch error.  mapping: 1 row-group, 2 merge path
// (main pass; the fix-up is launched separately).
hipError_t launch_spmm(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
// SpMM + SDDMM on one pattern sharing the gathered rows (fp32; row-group and
// merge-path mappings; split rows then go through launch_spmm_fixup)
hipError_t launch_dual(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_spmm_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s);
// row-group SpMM with wide lanes (one row per wave, 4 floats per lane, nv passes)
hipError_t launch_spmm_wide(int nv, const Fp32Args& a, hipStream_t s);
hipError_t launch_attention(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_attention_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s);
hipError_t launch_sddmm(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
// the same main kernels over bf16 gathered (and SDDMM row) operands, vec = 2, 4, 8
// bf16 values per lane; the fix-ups read fp32 pieces and are shared
hipError_t launch_spmm_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_sddmm_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_attention_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
// attention from queries and keys in one pass (U = Q, X = K, V = values)
hipError_t launch_attention_qk(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_attention_qk_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s);
hipError_t launch_attention_qk_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s);
// degree classes: the SpMM of the packed short rows (T = float or bf16 by
// dtype; vec, nv the lane layout of one row), and the construction
hipError_t launch_bucket_spmm(int dtype_bf16, int vec, int nv, const BucketArgs& a, hipStream_t s);
hipError_t bucket_build_workspace(int64_t n_rows, int64_t nnz, size_t* bytes);
// rows: the packed rows (stable by class), slot_col / slot_pos, long_row_ptr,
// long_col / long_pos of the rows with at least E entries or none;
// cls_* as in BucketArgs.
hipError_t launch_bucket_build(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t nnz, int E,
                               int n_classes, const int64_t* cls_rows, const int64_t* cls_base,
                               const int64_t* cls_row0, int32_t* rows, int32_t* slot_col, int32_t* slot_pos,
                               int32_t* long_row_ptr, int32_t* long_col, int32_t* long_pos, void* ws,
                               size_t ws_bytes, hipStream_t s);
// dst[k] = pos[k] >= 0 ? (src ? src[pos[k]] : 1) : 0 for k < n
hipError_t launch_gather_or_zero(const int32_t* pos, const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_mha(int mapping, int lph, int chunk, const MhaArgs& a, hipStream_t s);
hipError_t launch_mha_fixup(int lph, const MhaArgs& a, hipStream_t s);

hipError_t launch_row_softmax(int mapping, int chunk, const SoftmaxArgs& a, hipStream_t s);
hipError_t launch_row_softmax_backward(int chunk, const SoftmaxArgs& a, hipStream_t s);

// CSR of A^T (entries of each column in row order) and its entry permutation;
// the workspace holds two int32 [nnz] arrays and the sort's temporary storage.
hipError_t transpose_workspace(int64_t n_cols, int64_t nnz, size_t* bytes);
hipError_t launch_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t n_cols,
                            int64_t nnz, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm, void* ws,
                            size_t ws_bytes, hipStream_t s);
hipError_t launch_gather_values(const int32_t* perm, const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_invert(const int32_t* perm, int32_t* inv, int64_t n, hipStream_t s);
hipError_t permutation_plan_workspace(int64_t n, size_t* bytes);
hipError_t launch_permutation_plan(const int32_t* q, int64_t n, int wbits, int32_t* q1, int32_t* pos, void* ws,
                                   size_t ws_bytes, hipStream_t s);
hipError_t launch_permute(const int32_t* q1, const int32_t* pos, const float* src, float* tmp, float* dst, int64_t n,
                          hipStream_t s);
// the COO row array: rows[e] = the row holding entry e
hipError_t launch_coo_rows(const int32_t* row_ptr, int64_t n_rows, int32_t* rows, int64_t nnz, hipStream_t s);

// column-part segment format (k_hybrid.hip): construction in two steps (the
// sort, which reads the segment count back into pinned host memory, then the
// segment arrays); and (k_spmm.hip) the sum of each row's segment partial rows
// with the lane layout (vec, nv, W)
hipError_t hybrid_build_workspace(int64_t n_rows, int64_t nnz, int32_t parts, size_t* bytes);
hipError_t launch_hybrid_build_sort(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows, int64_t nnz,
                                    int32_t parts, int32_t part_cols, int32_t whole_below, int32_t* perm,
                                    int32_t* fcol, void* ws, size_t ws_bytes, int32_t* seg_count_host, hipStream_t s);
hipError_t launch_hybrid_build_segments(int64_t n_rows, int64_t nnz, int32_t parts, int64_t n_seg, int32_t* seg_ptr,
                                        int32_t* seg_row, int32_t* row_seg_ptr, int32_t* row_seg, void* ws,
                                        hipStream_t s);
hipError_t launch_hybrid_reduce(int vec, int nv, int W, float* Y, int64_t ldy, const float* part, int32_t F,
                                const int32_t* row_seg_ptr, const int32_t* row_seg, int64_t n_rows, hipStream_t s);

// Structure kernels.
hipError_t launch_fill_i64(int64_t* p, int64_t n, int64_t value, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t s);
hipError_t launch_degree_hist(const int32_t* row_ptr, int64_t n_rows, int64_t* out, hipStream_t s);
hipError_t launch_merge_path(const int32_t* row_ptr, int64_t n_rows, int64_t nnz, int64_t items,
                             int64_t n_chunks, int32_t* coords, hipStream_t s, int32_t* bounds = nullptr);
hipError_t launch_validate(const int32_t* row_ptr, const int32_t* col_idx, int64_t n_rows,
                           int64_t n_cols, int64_t nnz, int64_t* bad, hipStream_t s);
// Adds the count of idx[0 .. n) outside [0, bound) to *bad (not zeroed here).
hipError_t launch_validate_index(const int32_t* idx, int64_t n, int64_t bound, int64_t* bad, hipStream_t s);

} // namespace csrk
