// CSR SpMM kernels: Y = A X (row-group and merge-path mappings, fix-up).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_spmm(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Spmm>(mapping, vec, nv, chunk, a, s);
}
hipError_t launch_spmm_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s)
{
    return dispatch_fixup<Op::Spmm>(vec, nv, a, s);
}
} // namespace csrk
