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
  // units (group, b, h) padded to a multiple of 8: see the kernel's XCD mapping
  const int64_t units = (int64_t)a.G * a.B * a.H;
  const int64_t total = (units + 7) / 8 * 8 * a.n_qtiles;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)total), block(kThreads);
  if (a.qk_fp8) {
    if (a.D == 128) hipLaunchKernelGGL((attn_bf16_kernel<128, false, true, true>), grid, block, 0, stream, a);
    else if (a.D == 64) hipLaunchKernelGGL((attn_bf16_kernel<64, false, true, true>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.D == 128) hipLaunchKernelGGL((attn_bf16_kernel<128, false, false, true>), grid, block, 0, stream, a);
    else if (a.D == 64) hipLaunchKernelGGL((attn_bf16_kernel<64, false, false, true>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace as
