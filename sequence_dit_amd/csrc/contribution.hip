// Partition contribution: per query row, the weight of every partition in the
// composed output, and per group of rows the mean weight.
//   DiTango review page (pith.science), free-parameter ledger and Fig. 8 caption,
//   Eq. 8: partition importance w(i, t) is the softmax over partitions of LSE_t(i).
//
// Launch 1: one thread per row (256 rows per workgroup); LSE[i][row] reads are
// coalesced across threads (partition-major layout). Per row, M = max_i L_i and
// S = sum_i e^(L_i - M) in index order, then w_i = e^(L_i - M) / S: differences
// of nearby LSE values are exact, so w keeps fp32 accuracy whatever the size of
// the LSE values (forming L* = M + ln S first would round L* to the ulp of M).
// w is optionally written; for scores, the w of 32 partitions x 256 rows go
// through LDS and are summed in a fixed order (32-row runs, then the 8 runs) into
// one partial per (group, chunk, i) in the caller's workspace.
// Launch 2: one wave per (group, i) adds the chunk partials (lane-strided, then a
// butterfly). No atomics, so scores are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

constexpr int kThreads = kContribChunk;  // one row per thread
constexpr int kPB = 32;                  // partitions per LDS block
constexpr int kRun = kThreads / 8;       // rows summed by one thread: 8 runs of 32 per partition
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kThreads == 256, "8 runs of 32 rows");

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// e^(l - M) for l <= M (l = -inf gives 0)
__device__ __forceinline__ float rel_exp(float l, float M) { return __builtin_amdgcn_exp2f((l - M) * kLog2e); }

__global__ __launch_bounds__(kThreads) void contribution_rows_kernel(const ContribArgs a) {
  __shared__ float wt[kPB][kThreads + 1];   // w of one partition block, padded rows
  __shared__ float runs[8][kPB];
  const int g = blockIdx.x / a.chunks_per_group;
  const int chunk = blockIdx.x % a.chunks_per_group;
  const int t = threadIdx.x;
  const int64_t local = (int64_t)chunk * kThreads + t;
  const bool on = local < a.rows_per_group;
  const int64_t rows = a.rows;
  const int64_t row = (int64_t)g * a.rows_per_group + local;
  const float* lse = a.lse + row;   // LSE of partition i at lse[i * rows]
  const int P = a.P;

  float M = -INFINITY;
  if (on) {
#pragma unroll 8
    for (int i = 0; i < P; ++i) M = fmaxf(M, lse[i * rows]);
  }
  const bool live = on && M != -INFINITY;
  float S = 0.f;
  if (live) {
#pragma unroll 8
    for (int i = 0; i < P; ++i) S += rel_exp(lse[i * rows], M);
  }
  const float inv = live ? 1.0f / S : 0.f;

  for (int i0 = 0; i0 < P; i0 += kPB) {
    const int nb = P - i0 < kPB ? P - i0 : kPB;
    for (int j = 0; j < nb; ++j) {
      const int64_t i = i0 + j;
      const float w = live ? rel_exp(lse[i * rows], M) * inv : 0.f;
      if (on && a.weights) a.weights[i * rows + row] = w;
      wt[j][t] = w;
    }
    if (a.partial) {
      __syncthreads();
      const int j = t % kPB, r0 = (t / kPB) * kRun;   // partition i0 + j, rows r0 .. r0 + 31
      if (j < nb) {
        float x = 0.f;
#pragma unroll 8
        for (int r = 0; r < kRun; ++r) x += wt[j][r0 + r];
        runs[t / kPB][j] = x;
      }
      __syncthreads();
      if (t < nb) {
        float x = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) x += runs[q][t];
        a.partial[((int64_t)g * a.chunks_per_group + chunk) * P + i0 + t] = x;
      }
      __syncthreads();   // wt and runs are rewritten by the next block
    }
  }
}

__global__ __launch_bounds__(256) void contribution_groups_kernel(const ContribArgs a) {
  const int64_t G = a.rows / a.rows_per_group;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (group, partition)
  const int lane = threadIdx.x & 63;
  if (pair >= G * a.P) return;   // the whole wave leaves together
  const int64_t g = pair / a.P;
  const int i = (int)(pair % a.P);
  const float* part = a.partial + g * a.chunks_per_group * a.P + i;
  float t = 0.f;
  for (int c = lane; c < a.chunks_per_group; c += 64) t += part[(int64_t)c * a.P];
  t = wave_sum(t);
  if (lane == 0) a.scores[g * a.P + i] = t / (float)a.rows_per_group;
}

}  // namespace

hipError_t launch_contribution(const ContribArgs& a, hipStream_t stream) {
  const int64_t G = a.rows / a.rows_per_group;
  const int64_t blocks1 = G * a.chunks_per_group;
  if (blocks1 <= 0) return hipSuccess;
  if (blocks1 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(contribution_rows_kernel, dim3((unsigned)blocks1), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.scores) return e;
  const int64_t blocks2 = (G * a.P + 3) / 4;
  if (blocks2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(contribution_groups_kernel, dim3((unsigned)blocks2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
