// Grouped partition attention: launcher of the MFMA kernel of attn_kernel.h with its
// GROUPED flag. A workgroup walks the partitions of one group and writes the group's
// composed state (optionally composed with a given cached state), plus every
// partition's LSE.
//   DiTango review page (pith.science), axiom ledger (Eq. 1-2): states compose
//   associatively and commutatively; "If this is right": composed states merged into
//   coarser groups; referee report, summary: ring-based attention composition and
//   memory-aware state merging.
#include "attn_kernel.h"

namespace as {

namespace {
__global__ __launch_bounds__(256) void fill_neg_inf_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = -INFINITY;
}
}  // namespace

hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fill_neg_inf_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t stream) {
  if (a.v_fp8) return launch_attn_grouped_fp8v(a, stream);
  const int64_t total = attn_grid(a, true);
  if (total == 0) return hipSuccess;
  if (total < 0) return hipErrorInvalidConfiguration;
  if (a.qk_fp8) return launch_variant<true, true, false>(a, dim3((unsigned)total), stream);
  return launch_variant<false, true, false>(a, dim3((unsigned)total), stream);
}

}  // namespace as
