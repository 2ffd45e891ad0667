// CSR SpMM over bf16 features (raw bit patterns widened to fp32 in registers,
// fp32 accumulation and output): the row-group, merge-path and segmented-scan
// mappings of k_spmm.hip instantiated for 2, 4 or 8 bf16 values per lane.
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_spmm_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Spmm, bf16_t>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
