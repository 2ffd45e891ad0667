// CSR SpMM kernels: Y = A X (row-group and merge-path mappings, fix-up), and the sum of the column-part
// segment format's partial rows.
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_spmm(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Spmm, float>(mapping, vec, nv, chunk, a, s);
}
hipError_t launch_spmm_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s)
{
    return dispatch_fixup<Op::Spmm>(vec, nv, a, s);
}

template <int NV>
static hipError_t run_wide(const Fp32Args& a, hipStream_t s)
{
    constexpr int U = unroll_for(4, NV);
    const int64_t blocks = (a.n_rows * CSR_WAVE + CSR_BLOCK - 1) / CSR_BLOCK;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_rowgroup_wide<NV, U>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_spmm_wide(int nv, const Fp32Args& a, hipStream_t s)
{
    if (a.F < 4 || (int64_t)nv * CSR_WAVE * 4 < a.F) return hipErrorInvalidValue;
#define CSR_CASE(V, N) \
    if (nv == N) return run_wide<N>(a, s);
    CSR_NV_CASES(CSR_CASE, 4)
#undef CSR_CASE
    return hipErrorInvalidValue;
}
template <int VEC, int NV>
static hipError_t run_hyb_reduce(int W, float* Y, int64_t ldy, const float* part, int32_t F,
                                 const int32_t* row_seg_ptr, const int32_t* row_seg, int64_t n_rows, hipStream_t s)
{
    const int64_t blocks = (n_rows * W + CSR_BLOCK - 1) / CSR_BLOCK;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_hyb_reduce_rows<VEC, NV>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, Y, ldy, part, F, W,
                       row_seg_ptr, row_seg, n_rows);
    return hipGetLastError();
}

hipError_t launch_hybrid_reduce(int vec, int nv, int W, float* Y, int64_t ldy, const float* part, int32_t F,
                                const int32_t* row_seg_ptr, const int32_t* row_seg, int64_t n_rows, hipStream_t s)
{
#define CSR_CASE(V, N) \
    if (vec == V && nv == N) return run_hyb_reduce<V, N>(W, Y, ldy, part, F, row_seg_ptr, row_seg, n_rows, s);
    CSR_NV_CASES(CSR_CASE, 1)
    CSR_NV_CASES(CSR_CASE, 2)
    CSR_NV_CASES(CSR_CASE, 4)
#undef CSR_CASE
    return hipErrorInvalidValue;
}
} // namespace csrk
