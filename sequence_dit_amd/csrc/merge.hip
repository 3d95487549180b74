// Composition of attention states: n (OUT, LSE) pairs -> one (OUT, LSE).
//   DiTango review page (pith.science), axiom ledger, Eq. 1-2: states compose
//   associatively and commutatively (the online-softmax identity); "What carries
//   the argument": several remote partitions are merged into one cached state and
//   folded into the output later.
//
// The kernels are HBM-bound: every byte of every input is read once, every output
// byte written once. One thread owns one 16-byte chunk (4 floats) of one row, so a
// wave reads 1 KB contiguous per input per load instruction. Inputs whose weight
// is exactly zero (empty states) are neither read nor added, and the accumulator
// starts at -0.0 (the additive identity of IEEE arithmetic), so composing any
// state with empty states returns it bit for bit.
//
// merge_rows_kernel (D = 32, 64, 128, 256) loads each row's LSE values once and
// shares the weights through LDS; merge_kernel is the general path (any D that is
// a multiple of 4), where every lane of a row reads the row's LSE values.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeArgs a) {
  const int cpr = a.D >> 2;  // 16-byte chunks per row
  const int64_t total = a.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kMergeThreads;
  for (int64_t c = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x; c < total; c += stride) {
    const int64_t row = c / cpr;
    const int col = (int)(c - row * cpr);
    float M = -INFINITY;
    for (int k = 0; k < a.n; ++k) M = fmaxf(M, a.lses[k][row]);
    const int64_t off = row * a.D + 4 * col;
    if (M == -INFINITY) {  // every input empty: the empty state
      *reinterpret_cast<f32x4*>(a.out + off) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (col == 0) a.lse[row] = -INFINITY;
      continue;
    }
    f32x4 acc = {-0.f, -0.f, -0.f, -0.f};
    float S = 0.f;
    int k = 0;
    for (; k + 4 <= a.n; k += 4) {
      float w[4];
      f32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = expf(a.lses[k + j][row] - M);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[j] = (w[j] != 0.f) ? *reinterpret_cast<const f32x4*>(a.outs[k + j] + off) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (w[j] != 0.f) {
          S += w[j];
          acc[0] = __builtin_fmaf(w[j], x[j][0], acc[0]);
          acc[1] = __builtin_fmaf(w[j], x[j][1], acc[1]);
          acc[2] = __builtin_fmaf(w[j], x[j][2], acc[2]);
          acc[3] = __builtin_fmaf(w[j], x[j][3], acc[3]);
        }
      }
    }
    for (; k < a.n; ++k) {
      const float w = expf(a.lses[k][row] - M);
      if (w != 0.f) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.outs[k] + off);
        S += w;
        acc[0] = __builtin_fmaf(w, x[0], acc[0]);
        acc[1] = __builtin_fmaf(w, x[1], acc[1]);
        acc[2] = __builtin_fmaf(w, x[2], acc[2]);
        acc[3] = __builtin_fmaf(w, x[3], acc[3]);
      }
    }
    const f32x4 r = {acc[0] / S, acc[1] / S, acc[2] / S, acc[3] / S};
    *reinterpret_cast<f32x4*>(a.out + off) = r;
    if (col == 0) a.lse[row] = M + logf(S);
  }
}


// Fast path for D/4 = CPR in {8, 16, 32, 64} chunks per row: a wave owns 64/CPR rows;
// the n LSE values of a row are loaded once (one per lane of the row group), the
// row's max, weights and their sum are reduced within the group, and the weights
// are handed to the row's lanes through LDS (broadcast reads), so the streaming
// loop issues only the OUT loads, with nontemporal hints (the inputs are read once).
template <int CPR>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_kernel(const MergeArgs a) {
  constexpr int RPW = 64 / CPR;                 // rows per wave
  constexpr int RPB = RPW * (kMergeThreads / 64);
  __shared__ float wsh[kMergeThreads / 64][RPW][AS_MAX_MERGE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / CPR, j = lane % CPR;     // row within the wave, lane within the row
  const int64_t row = (int64_t)blockIdx.x * RPB + wave * RPW + g;
  const bool live = row < a.rows;
  // 1. LSE of inputs j, j + CPR, ... of this row; max over the row group
  float Lv[AS_MAX_MERGE / CPR > 0 ? AS_MAX_MERGE / CPR : 1];
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < AS_MAX_MERGE / CPR; ++u) {
    const int k = j + u * CPR;
    Lv[u] = (live && k < a.n) ? a.lses[k][row] : -INFINITY;
    M = fmaxf(M, Lv[u]);
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, CPR));
  const bool empty = (M == -INFINITY);
  float S = 0.f;
#pragma unroll
  for (int u = 0; u < AS_MAX_MERGE / CPR; ++u) {
    const int k = j + u * CPR;
    const float w = empty ? 0.f : expf(Lv[u] - M);
    S += w;
    if (k < AS_MAX_MERGE) wsh[wave][g][k] = w;
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) S += __shfl_xor(S, m, CPR);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  if (!live) return;
  const int64_t off = row * a.D + 4 * j;
  if (empty) {
    *reinterpret_cast<f32x4*>(a.out + off) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j == 0) a.lse[row] = -INFINITY;
    return;
  }
  // 2. stream the inputs with non-zero weight
  f32x4 acc = {-0.f, -0.f, -0.f, -0.f};
  int k = 0;
  for (; k + 4 <= a.n; k += 4) {
    float w[4];
    f32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = wsh[wave][g][k + u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = (w[u] != 0.f) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.outs[k + u] + off))
                           : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (w[u] != 0.f) {
        acc[0] = __builtin_fmaf(w[u], x[u][0], acc[0]);
        acc[1] = __builtin_fmaf(w[u], x[u][1], acc[1]);
        acc[2] = __builtin_fmaf(w[u], x[u][2], acc[2]);
        acc[3] = __builtin_fmaf(w[u], x[u][3], acc[3]);
      }
  }
  for (; k < a.n; ++k) {
    const float w = wsh[wave][g][k];
    if (w != 0.f) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.outs[k] + off));
      acc[0] = __builtin_fmaf(w, x[0], acc[0]);
      acc[1] = __builtin_fmaf(w, x[1], acc[1]);
      acc[2] = __builtin_fmaf(w, x[2], acc[2]);
      acc[3] = __builtin_fmaf(w, x[3], acc[3]);
    }
  }
  const f32x4 r = {acc[0] / S, acc[1] / S, acc[2] / S, acc[3] / S};
  __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(a.out + off));
  if (j == 0) a.lse[row] = M + logf(S);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t total = a.rows * (a.D / 4);
  if (total <= 0) return hipSuccess;
  const int cpr = a.D / 4;
  if (cpr == 8 || cpr == 16 || cpr == 32 || cpr == 64) {
    const int64_t rpb = (64 / cpr) * (kMergeThreads / 64);
    const dim3 grid((unsigned)((a.rows + rpb - 1) / rpb)), block(kMergeThreads);
    switch (cpr) {
      case 8: hipLaunchKernelGGL(merge_rows_kernel<8>, grid, block, 0, stream, a); break;
      case 16: hipLaunchKernelGGL(merge_rows_kernel<16>, grid, block, 0, stream, a); break;
      case 32: hipLaunchKernelGGL(merge_rows_kernel<32>, grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL(merge_rows_kernel<64>, grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
  }
  int64_t blocks = (total + kMergeThreads - 1) / kMergeThreads;
  if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;  // grid-stride beyond this
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
