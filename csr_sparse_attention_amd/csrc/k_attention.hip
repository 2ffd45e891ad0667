// Fused CSR softmax attention with given edge scores (row-group and
// merge-path mappings, (max, sum, acc) fix-up).
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_attention(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::Attention, float>(mapping, vec, nv, chunk, a, s);
}
hipError_t launch_attention_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s)
{
    return dispatch_fixup<Op::Attention>(vec, nv, a, s);
}
} // namespace csrk
