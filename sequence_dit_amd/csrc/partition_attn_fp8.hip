// Partition attention with fp8 E4M3 queries and keys: launcher of the MFMA kernel of
// attn_kernel.h with its QK8 flag (S = K Q^T on the fp8 MFMA, softmax and PV as for bf16).
//   DiTango review page (pith.science), reference list: SageAttention (8-bit attention
//   for inference); FastUSP page (mlsanity), prior work: the FP8 formats paper (E4M3).
#include "attn_kernel.h"

namespace as {

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream) {
  if (a.v_fp8) return launch_attn_fp8v(a, stream);
  const int64_t total = attn_grid(a, false);
  if (total == 0) return hipSuccess;
  if (total < 0) return hipErrorInvalidConfiguration;
  return launch_variant<true, false, false>(a, dim3((unsigned)total), stream);
}

}  // namespace as
