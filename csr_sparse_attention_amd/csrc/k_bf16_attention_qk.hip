// CSR attention from bf16 queries, keys and values in one pass (fp32
// accumulation); the fix-up is the fp32 one of k_attention_qk.hip.
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_attention_qk_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::AttnQK, bf16_t>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
