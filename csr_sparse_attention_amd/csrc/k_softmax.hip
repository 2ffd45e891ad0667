// Standalone CSR row softmax (statistics and in-chunk normalisation,
// split-row merge, split-row normalisation).
#include "launch.h"
#include "softmax_kernels.h"

namespace csrk {

template <int D>
static hipError_t run_softmax(const SoftmaxArgs& a, hipStream_t s)
{
    const int64_t blocks = (a.n_chunks + CSR_WAVES_PER_BLOCK - 1) / CSR_WAVES_PER_BLOCK;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_softmax_main<D>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t fblocks = (a.n_chunks + CSR_WAVE * CSR_WAVES_PER_BLOCK - 1) / (CSR_WAVE * CSR_WAVES_PER_BLOCK);
    hipLaunchKernelGGL(k_softmax_fixup, dim3((unsigned)fblocks), dim3(CSR_BLOCK), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_softmax_split, dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_row_softmax(int chunk, const SoftmaxArgs& a, hipStream_t s)
{
    switch (chunk) {
    case 256: return run_softmax<256>(a, s);
    case 512: return run_softmax<512>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csrk
