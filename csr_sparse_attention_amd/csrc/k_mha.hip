// Multi-head fused CSR attention (bf16 Q/K/V, fp32 accumulation).
#include "launch.h"
#include "mha_kernels.h"

namespace csrk {

template <int LPH>
static hipError_t run_mha(int mapping, int chunk, const MhaArgs& a, hipStream_t s)
{
    constexpr int U = 8;  // entries in flight per wavefront
    if (mapping == 1) {
        const int64_t blocks = (a.n_rows + CSR_WAVES_PER_BLOCK - 1) / CSR_WAVES_PER_BLOCK;
        if (blocks == 0) return hipSuccess;
        hipLaunchKernelGGL((k_mha_rowgroup<LPH, U>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
        return hipGetLastError();
    }
    const int64_t blocks = (a.n_chunks + CSR_WAVES_PER_BLOCK - 1) / CSR_WAVES_PER_BLOCK;
    if (blocks == 0) return hipSuccess;
    switch (chunk) {
    case 256: hipLaunchKernelGGL((k_mha_mergepath<LPH, U, 256>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a); break;
    case 512: hipLaunchKernelGGL((k_mha_mergepath<LPH, U, 512>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k_mha_mergepath<LPH, U, 1024>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int LPH>
static hipError_t run_mha_fixup(const MhaArgs& a, hipStream_t s)
{
    const int64_t blocks = (a.n_chunks + CSR_WAVE * CSR_WAVES_PER_BLOCK - 1) / (CSR_WAVE * CSR_WAVES_PER_BLOCK);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_mha_fixup<LPH>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    return hipGetLastError();
}

#define CSR_LPH_CASES(M) M(1) M(2) M(4) M(8) M(16) M(32) M(64)

hipError_t launch_mha(int mapping, int lph, int chunk, const MhaArgs& a, hipStream_t s)
{
#define CSR_CASE(L) if (lph == L) return run_mha<L>(mapping, chunk, a, s);
    CSR_LPH_CASES(CSR_CASE)
#undef CSR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_mha_fixup(int lph, const MhaArgs& a, hipStream_t s)
{
#define CSR_CASE(L) if (lph == L) return run_mha_fixup<L>(a, s);
    CSR_LPH_CASES(CSR_CASE)
#undef CSR_CASE
    return hipErrorInvalidValue;
}

} // namespace csrk
