// Partition attention with fp8 E4M3 queries, keys and values: launchers of the MFMA kernel
// of attn_kernel.h with its QK8 and V8 flags, single-partition and grouped. V's codes are
// widened to bf16 on their way into LDS (exactly) and V's per-(b, h) factor scales OUT in
// the epilogue, so only the HBM bytes of V change.
//   FastUSP page (mlsanity), abstract: attention traffic quantised to FP8; prior work:
//   the FP8 formats paper (E4M3). DiTango review page (pith.science), reference list:
//   SageAttention (8-bit attention for inference).
#include "attn_kernel.h"

namespace as {

hipError_t launch_attn_fp8v(const AttnArgs& a, hipStream_t stream) {
  const int64_t total = attn_grid(a, false);
  if (total == 0) return hipSuccess;
  if (total < 0) return hipErrorInvalidConfiguration;
  return launch_variant<true, false, true>(a, dim3((unsigned)total), stream);
}

hipError_t launch_attn_grouped_fp8v(const AttnArgs& a, hipStream_t stream) {
  const int64_t total = attn_grid(a, true);
  if (total == 0) return hipSuccess;
  if (total < 0) return hipErrorInvalidConfiguration;
  return launch_variant<true, true, true>(a, dim3((unsigned)total), stream);
}

}  // namespace as
