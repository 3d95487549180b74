// Composition of attention states: n (OUT, LSE) pairs -> one (OUT, LSE).
//   DiTango review page (pith.science), axiom ledger, Eq. 1-2: states compose
//   associatively and commutatively (the online-softmax identity); "What carries
//   the argument": several remote partitions are merged into one cached state and
//   folded into the output later.
//
// The kernel is HBM-bound: every byte of every input is read once, every output
// byte written once. One thread owns one 16-byte chunk (4 floats) of one row, so a
// wave reads 1 KB contiguous per input per load instruction; the n LSE loads of a
// row are broadcast reads shared by the row's D/4 lanes. Inputs whose weight is
// exactly zero (empty states) are neither read nor added, and the accumulator
// starts at -0.0 (the additive identity of IEEE arithmetic), so composing any
// state with empty states returns it bit for bit.
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

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t total = a.rows * (a.D / 4);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + kMergeThreads - 1) / kMergeThreads;
  if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;  // grid-stride beyond this
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
