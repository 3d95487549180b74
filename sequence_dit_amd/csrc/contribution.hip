// Partition contribution: per query row, the weight of every partition in the
// composed output, and per group of rows the mean weight.
//   DiTango review page (pith.science), free-parameter ledger and Fig. 8 caption,
//   Eq. 8: partition importance w(i, t) is the softmax over partitions of LSE_t(i).
//
// Launch 1: one thread per row (256 rows per workgroup); LSE[i][row] reads are
// coalesced across threads (partition-major layout); up to 32 partitions the row's LSE
// values are read once into registers, above that in blocks of 32 (two passes). Per row,
// M = max_i L_i and S = sum_i e^(L_i - M) (in index order up to 32 partitions; above, per
// block, rescaled when a block moves the max), then w_i = e^(L_i - M) / S: differences
// of nearby LSE values are exact, so w keeps fp32 accuracy whatever the size of
// the LSE values (forming L* = M + ln S first would round L* to the ulp of M).
// w is optionally written; for scores, the w of 32 partitions x 256 rows go
// through LDS and are summed in a fixed order (32-row runs, then the 8 runs) into
// one partial per (group, chunk, i) in the caller's workspace (for the
// allocation-free entry point, in the library's static scratch instead).
// Launch 2: one wave per (group, i) adds the chunk partials (lane-strided, then a
// butterfly). No atomics, so scores are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "as_internal.h"

// Partial sums of the allocation-free entry point (as_partition_contribution_noalloc):
// one copy per device, held until the process ends. Host code must not pass this
// name to a kernel (on the host it is only a stand-in for the device variable): the
// device address comes from contribution_scratch().
static __device__ __align__(256) float scratch[as::kContribScratchBytes / sizeof(float)];

namespace as {

hipError_t contribution_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    // once per device, with that device current: its own copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<float*>(p);
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

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

// PR > 0 (P <= PR): the row's P LSE values are loaded once, all in flight together, and
// kept in registers (the loops over partitions are unrolled to PR with a predicate; the sum
// runs in index order, adding exact zeros for i >= P). PR = 0 (any P): two passes over
// blocks of kPB partitions, each block loaded together; the first keeps the running max and
// a sum rescaled when a block moves it, the second gives the weights.
template <int PR>
__global__ __launch_bounds__(kThreads) void contribution_rows_kernel(const ContribArgs a) {
  static_assert(PR == 0 || PR <= kPB, "one LDS block of partitions");
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

  float L[PR > 0 ? PR : 1];
  float M = -INFINITY;
  if constexpr (PR > 0) {
#pragma unroll
    for (int i = 0; i < PR; ++i) L[i] = (on && i < P) ? lse[i * rows] : -INFINITY;
#pragma unroll
    for (int i = 0; i < PR; ++i) M = fmaxf(M, L[i]);
  }
  float S = 0.f;
  if constexpr (PR == 0) {
    // blocks of kPB partitions, each block's LSE values loaded together; the max and the sum
    // run over the blocks in one pass, the sum rescaled when a block moves the max
    if (on) {
      for (int i0 = 0; i0 < P; i0 += kPB) {
        float X[kPB];
#pragma unroll
        for (int j = 0; j < kPB; ++j) X[j] = i0 + j < P ? lse[(int64_t)(i0 + j) * rows] : -INFINITY;
        float mb = M;
#pragma unroll
        for (int j = 0; j < kPB; ++j) mb = fmaxf(mb, X[j]);
        if (mb != -INFINITY) {
          S *= rel_exp(M, mb);   // 1 when the max stays, 0 before the first finite value
          M = mb;
#pragma unroll
          for (int j = 0; j < kPB; ++j) S += rel_exp(X[j], M);
        }
      }
    }
  }
  const bool live = on && M != -INFINITY;
  if constexpr (PR > 0) {
    if (live) {
#pragma unroll
      for (int i = 0; i < PR; ++i) S += rel_exp(L[i], M);
    }
  }
  const float inv = live ? 1.0f / S : 0.f;

  for (int i0 = 0; i0 < P; i0 += kPB) {
    const int nb = P - i0 < kPB ? P - i0 : kPB;
    if constexpr (PR > 0) {
#pragma unroll
      for (int j = 0; j < PR; ++j) {
        if (j < nb) {
          const float w = live ? rel_exp(L[j], M) * inv : 0.f;
          if (on && a.weights) a.weights[(int64_t)j * rows + row] = w;
          wt[j][t] = w;
        }
      }
    } else {
      float X[kPB];
#pragma unroll
      for (int j = 0; j < kPB; ++j) X[j] = (live && j < nb) ? lse[(int64_t)(i0 + j) * rows] : -INFINITY;
#pragma unroll
      for (int j = 0; j < kPB; ++j) {
        if (j < nb) {
          const float w = live ? rel_exp(X[j], M) * inv : 0.f;
          if (on && a.weights) a.weights[(int64_t)(i0 + j) * rows + row] = w;
          wt[j][t] = w;
        }
      }
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
  if (a.P <= 8) hipLaunchKernelGGL(contribution_rows_kernel<8>, dim3((unsigned)blocks1), dim3(kThreads), 0, stream, a);
  else if (a.P <= kPB) hipLaunchKernelGGL(contribution_rows_kernel<kPB>, dim3((unsigned)blocks1), dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(contribution_rows_kernel<0>, dim3((unsigned)blocks1), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.scores) return e;
  const int64_t blocks2 = (G * a.P + 3) / 4;
  if (blocks2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(contribution_groups_kernel, dim3((unsigned)blocks2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
