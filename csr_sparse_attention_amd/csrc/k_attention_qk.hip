// CSR attention from fp32 queries and keys in one pass (SDDMM -> row-softmax
// -> SpMM with the scores formed on the fly and folded into an online
// softmax): row-group and merge-path mappings, (max, sum, acc) fix-up.
#include "launch.h"
#include "fp32_kernels.h"
#include "fp32_launch.inc"

namespace csrk {
hipError_t launch_attention_qk(int mapping, int vec, int nv, int chunk, const Fp32Args& a, hipStream_t s)
{
    return dispatch_main<Op::AttnQK, float>(mapping, vec, nv, chunk, a, s);
}
hipError_t launch_attention_qk_fixup(int vec, int nv, const Fp32Args& a, hipStream_t s)
{
    return dispatch_fixup<Op::AttnQK>(vec, nv, a, s);
}
} // namespace csrk
