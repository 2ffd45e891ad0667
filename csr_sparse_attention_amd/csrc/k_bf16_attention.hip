// Fused CSR softmax attention with given fp32 edge scores over bf16 node
// values (fp32 accumulation and output).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_attention_bf16(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Attention, bf16_t>(mapping, vec, nv, chunk, a, s);
}
} // namespace csrk
