// Partition attention: launchers of the MFMA kernel for bf16 inputs (attn_kernel.h) and the
// fp32 accuracy path.
//   DiTango review page (pith.science), "What carries the argument": the state of a
//   partition is its partial attention output with the log-sum-exp of its scores.
#include "attn_kernel.h"

namespace as {
namespace {

// ------------------------------------------------------------------------------
// fp32 accuracy path: one workgroup = 64 query rows (4 lanes per row, each lane
// owning D/4 of the head dimension) x one (batch, head) x one partition. K/V tiles
// of 32 keys are staged in LDS; scores and the online softmax are fp32 with the
// natural-base exponential.
// ------------------------------------------------------------------------------
constexpr int kF32Rows = 64;
constexpr int kF32Threads = 256;
constexpr int kF32Keys = 32;

template <int DC, bool OUT_BF16>  // D / 4 elements per lane (1..32)
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(const AttnArgs a) {
  const int D = a.D;
  __shared__ float ks_[kF32Keys][128 + 4];
  __shared__ float vs_[kF32Keys][128 + 4];

  const int bhp = blockIdx.y;
  const int bh = bhp % (a.B * a.H);
  const int part = bhp / (a.B * a.H);
  const int b = bh / a.H, hh = bh % a.H;
  const int tid = threadIdx.x;
  const int rloc = tid >> 2, sub = tid & 3;
  const int q = blockIdx.x * kF32Rows + rloc;
  const int ksb = a.ranges[2 * part], keb = a.ranges[2 * part + 1];
  const int n = keb - ksb;
  const int64_t row_base = ((int64_t)part * a.B * a.H + bh) * a.Sq;
  float* lse = a.lse + row_base;
  const int dc = D / 4;   // elements per lane

  float qv[DC], acc[DC];
  const float* qp = reinterpret_cast<const float*>(a.q) + b * a.q_sb + hh * a.q_sh;
#pragma unroll
  for (int j = 0; j < DC; ++j) {
    qv[j] = (q < a.Sq && j < dc) ? qp[(int64_t)q * a.q_ss + sub * dc + j] : 0.f;
    acc[j] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kp = reinterpret_cast<const float*>(a.k) + b * a.k_sb + hh * a.k_sh;
  const float* vp = reinterpret_cast<const float*>(a.v) + b * a.k_sb + hh * a.k_sh;

  for (int key0 = 0; key0 < n; key0 += kF32Keys) {
    __syncthreads();
    for (int idx = tid; idx < kF32Keys * D; idx += kF32Threads) {
      const int r = idx / D, c = idx % D;
      const bool ok = key0 + r < n;
      const int64_t off = (int64_t)(ksb + key0 + r) * a.k_ss + c;
      ks_[r][c] = ok ? kp[off] : 0.f;
      vs_[r][c] = ok ? vp[off] : 0.f;
    }
    __syncthreads();
    const int cnt = min(kF32Keys, n - key0);
    float z[kF32Keys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < DC; ++e)
        if (e < dc) d = __builtin_fmaf(qv[e], ks_[j][sub * dc + e], d);
      d += __shfl_xor(d, 1, 4);
      d += __shfl_xor(d, 2, 4);
      z[j] = (j < cnt) ? d * a.scale : -INFINITY;
      tmax = fmaxf(tmax, z[j]);
    }
    const float mn = fmaxf(m, tmax);
    const float f = expf(m - mn);
    l *= f;
#pragma unroll
    for (int e = 0; e < DC; ++e) acc[e] *= f;
    m = mn;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      const float p = expf(z[j] - m);
      l += p;
#pragma unroll
      for (int e = 0; e < DC; ++e)
        if (e < dc) acc[e] = __builtin_fmaf(p, vs_[j][sub * dc + e], acc[e]);
    }
  }
  if (q < a.Sq) {
    if (n <= 0) {
      for (int e = 0; e < dc; ++e) store_out1<OUT_BF16>(a.out, (row_base + q) * D + sub * dc + e, 0.f);
      if (sub == 0) lse[q] = -INFINITY;
    } else {
      for (int e = 0; e < DC; ++e)
        if (e < dc) store_out1<OUT_BF16>(a.out, (row_base + q) * D + sub * dc + e, acc[e] / l);
      if (sub == 0) lse[q] = m + logf(l);
    }
  }
}

}  // namespace

int attn_bf16_rows_per_block(int) { return kBQ; }
int attn_f32_rows_per_block(int) { return kF32Rows; }

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.qk_fp8) return launch_attn_fp8(a, stream);
  const int64_t total = attn_grid(a, false);
  if (total == 0) return hipSuccess;
  if (total < 0) return hipErrorInvalidConfiguration;
  return launch_variant<false, false, false>(a, dim3((unsigned)total), stream);
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.out_kind != kOutF32 && a.out_kind != kOutBF16) return hipErrorInvalidValue;
  const int64_t gy = (int64_t)a.B * a.H * a.P;
  if (gy <= 0 || a.Sq <= 0) return hipSuccess;
  if (gy > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((a.Sq + kF32Rows - 1) / kF32Rows), (unsigned)gy), block(kF32Threads);
  const int dc = a.D / 4;
  if (dc <= 8) {
    if (a.out_kind == kOutBF16) hipLaunchKernelGGL((attn_f32_kernel<8, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<8, false>), grid, block, 0, stream, a);
  } else if (dc <= 16) {
    if (a.out_kind == kOutBF16) hipLaunchKernelGGL((attn_f32_kernel<16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<16, false>), grid, block, 0, stream, a);
  } else if (dc <= 32) {
    if (a.out_kind == kOutBF16) hipLaunchKernelGGL((attn_f32_kernel<32, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<32, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace as

#ifdef AS_WG_STAMPS
// Diagnostics build only: copies (or clears) the workgroup stamps of the single-partition
// bf16 kernels of this file; returns a hipError_t.
extern "C" int as_debug_wg_stamps(void* host, size_t bytes) {
  if (bytes > sizeof(as::as_wg_stamps)) bytes = sizeof(as::as_wg_stamps);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(as::as_wg_stamps), bytes);
}
extern "C" int as_debug_wg_stamps_clear() {
  static unsigned long long zeros[as::kStampWGs * 8];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(as::as_wg_stamps), zeros, sizeof(zeros));
}
#endif
