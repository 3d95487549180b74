// Partition attention with fp8 E4M3 queries and keys: launcher of the MFMA kernel of
// attn_kernel.h with its QK8 flag (S = K Q^T on the fp8 MFMA, softmax and PV as for bf16).
//   DiTango review page (pith.science), reference list: SageAttention (8-bit attention
//   for inference); FastUSP page (mlsanity), prior work: the FP8 formats paper (E4M3).
#include "attn_kernel.h"

namespace as {

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.n_qtiles * a.B * a.H * a.P;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)total), block(kThreads);
  if (a.D == 128) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<128, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, false, true>), grid, block, 0, stream, a);
  } else if (a.D == 64) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<64, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, false, true>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace as
