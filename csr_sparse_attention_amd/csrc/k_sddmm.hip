// CSR SDDMM kernels: out_e = <U[row_e], V[col_e]> (row-group and merge-path
// mappings; every entry is written by exactly one lane, no fix-up needed).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_sddmm(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Sddmm, float>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
