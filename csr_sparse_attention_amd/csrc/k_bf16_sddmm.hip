// CSR SDDMM over bf16 row operands U and V (fp32 accumulation and output).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_sddmm_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Sddmm, bf16_t>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
