// Partition contribution: per query row, the weight of every partition in the
// composed output, and per group of rows the mean weight.
//   DiTango review page (pith.science), free-parameter ledger and Fig. 8 caption,
//   Eq. 8: partition importance w(i, t) is the softmax over partitions of LSE_t(i).
//
// Launch 1: one thread per row; LSE[i][row] reads are coalesced across threads
// (partition-major layout). w is optionally written; for scores, each workgroup
// reduces its w[i] over its rows in a fixed order (wave butterfly, then waves in
// index order) into one partial per (group, chunk, i) in the caller's workspace.
// Launch 2: one thread per (group, i) sums its chunk partials in chunk order.
// No atomics, so scores are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

constexpr int kThreads = kContribChunk;  // one row per thread
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void contribution_rows_kernel(const ContribArgs a) {
  __shared__ float red[kWaves][AS_MAX_PARTITIONS];
  const int g = blockIdx.x / a.chunks_per_group;
  const int chunk = blockIdx.x % a.chunks_per_group;
  const int64_t local = (int64_t)chunk * kThreads + threadIdx.x;
  const bool on = local < a.rows_per_group;
  const int64_t row = (int64_t)g * a.rows_per_group + local;
  const float* lse = a.lse;
  const int64_t rows = a.rows;

  float M = -INFINITY;
  if (on)
    for (int i = 0; i < a.P; ++i) M = fmaxf(M, lse[i * rows + row]);
  float S = 0.f;
  if (on && M != -INFINITY)
    for (int i = 0; i < a.P; ++i) S += expf(lse[i * rows + row] - M);
  const bool live = on && M != -INFINITY;
  const float lstar = live ? M + logf(S) : 0.f;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = 0; i < a.P; ++i) {
    float w = 0.f;
    if (live) w = expf(lse[i * rows + row] - lstar);
    if (on && a.weights) a.weights[i * rows + row] = w;
    if (a.partial) {
      const float ws = wave_sum(w);
      if (lane == 0) red[wave][i] = ws;
    }
  }
  if (a.partial) {
    __syncthreads();
    for (int i = threadIdx.x; i < a.P; i += kThreads) {
      float t = 0.f;
      for (int wv = 0; wv < kWaves; ++wv) t += red[wv][i];
      a.partial[((int64_t)g * a.chunks_per_group + chunk) * a.P + i] = t;
    }
  }
}

__global__ __launch_bounds__(256) void contribution_groups_kernel(const ContribArgs a) {
  const int64_t G = a.rows / a.rows_per_group;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= G * a.P) return;
  const int64_t g = idx / a.P;
  const int i = (int)(idx % a.P);
  float t = 0.f;
  for (int c = 0; c < a.chunks_per_group; ++c) t += a.partial[(g * a.chunks_per_group + c) * a.P + i];
  a.scores[g * a.P + i] = t / (float)a.rows_per_group;
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
  const int64_t blocks2 = (G * a.P + 255) / 256;
  hipLaunchKernelGGL(contribution_groups_kernel, dim3((unsigned)blocks2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
