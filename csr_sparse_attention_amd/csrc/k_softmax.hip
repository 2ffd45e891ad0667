// Standalone CSR row softmax (statistics and in-chunk normalisation by row
// segments or by lane-owned entry runs, split-row merge, split-row
// normalisation).
#include "launch.h"
#include "softmax_kernels.h"

namespace csrk {

template <int D, bool RUNS, bool BWD = false>
static hipError_t run_softmax(const SoftmaxArgs& a, hipStream_t s)
{
    const int64_t blocks = (a.n_chunks + CSR_WAVES_PER_BLOCK - 1) / CSR_WAVES_PER_BLOCK;
    if (blocks == 0) return hipSuccess;
    if constexpr (RUNS)
        hipLaunchKernelGGL((k_softmax_run<D, BWD>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    else
        hipLaunchKernelGGL((k_softmax_main<D>), dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t fblocks =
        (a.n_chunks + SM_FIX_CHUNKS * CSR_WAVES_PER_BLOCK - 1) / (SM_FIX_CHUNKS * CSR_WAVES_PER_BLOCK);
    hipLaunchKernelGGL((k_softmax_fixup<BWD>), dim3((unsigned)fblocks), dim3(CSR_BLOCK), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (RUNS)
        hipLaunchKernelGGL((k_softmax_split_runs<BWD>), dim3((unsigned)fblocks), dim3(CSR_BLOCK), 0, s, a);
    else
        hipLaunchKernelGGL(k_softmax_split, dim3((unsigned)blocks), dim3(CSR_BLOCK), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_row_softmax(int mapping, int chunk, const SoftmaxArgs& a, hipStream_t s)
{
    if (mapping == CSR_MAP_SEGSCAN) {
        switch (chunk) {
        case 256: return run_softmax<256, true>(a, s);
        case 512: return run_softmax<512, true>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (chunk) {
    case 256: return run_softmax<256, false>(a, s);
    case 512: return run_softmax<512, false>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_row_softmax_backward(int chunk, const SoftmaxArgs& a, hipStream_t s)
{
    switch (chunk) {
    case 256: return run_softmax<256, true, true>(a, s);
    case 512: return run_softmax<512, true, true>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace csrk
