// SpMM and SDDMM on one CSR pattern sharing the gathered operand: Y = A X and
// z_e = <U[row_e], X[col_e]> from one read of each gathered row (row-group and
// merge-path mappings; the merge path's split rows are combined by the SpMM
// fix-up, whose carry layout this op shares).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_dual(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    if (mapping != 1 && mapping != 2) return hipErrorInvalidValue;
    return dispatch_main<Op::Dual, float>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
