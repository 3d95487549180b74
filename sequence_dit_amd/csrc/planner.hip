// Anchor-guided planner statistics.
//   DiTango review page (pith.science): "What carries the argument" (group error of
//   Eq. 12), free-parameter ledger (scale ratio of Eq. 9, group size, thresholds of
//   Algorithm 1) and the referee report on section 4.1.2 (drift model of Eq. 10,
//   reuse decision of Eq. 13).
//
// state_norms_partial_kernel / state_norms_final_kernel: L2 norms of P slices of n
// floats (or of slice differences). HBM-bound: every input byte is read once, with
// nontemporal 16-byte loads. Differences and squares of fp32 inputs are exact in
// fp64; only the sums round, and they are taken in a fixed order: per thread, then
// a wave butterfly, then the four waves in index order, then the chunks of a slice
// in a fixed order (eight lane-strided sums per lane, a tree, a butterfly). No atomics,
// so the norms are bitwise reproducible.
//
// planner_decide_kernel / planner_epsilon_kernel: one workgroup, one thread per
// partition (P <= 256); fp32 arithmetic on a few hundred scalars.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNormThreads = 256;

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <bool DIFF>
__global__ __launch_bounds__(kNormThreads) void state_norms_partial_kernel(const NormArgs a) {
  const int p = blockIdx.y;
  const int64_t c = blockIdx.x;
  const float* x = a.a + (int64_t)p * a.n;
  const float* y = DIFF ? a.b + (int64_t)p * a.n : nullptr;
  const int64_t start = c * a.chunk;
  const int64_t end = start + a.chunk < a.n ? start + a.chunk : a.n;
  // kUnroll 16-byte loads per input in flight per thread (guarded, so the last
  // iteration of a ragged chunk stays in bounds)
  constexpr int kUnroll = 4;
  constexpr int64_t kStep = 4 * kNormThreads;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (int64_t base = start + 4 * threadIdx.x; base < end; base += kUnroll * kStep) {
    f32x4 u[kUnroll], v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int64_t e = base + k * kStep;
      u[k] = e < end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + e)) : f32x4{0.f, 0.f, 0.f, 0.f};
      if (DIFF)
        v[k] = e < end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + e)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      double d0 = u[k][0], d1 = u[k][1], d2 = u[k][2], d3 = u[k][3];
      if (DIFF) {
        d0 -= v[k][0];
        d1 -= v[k][1];
        d2 -= v[k][2];
        d3 -= v[k][3];
      }
      s0 = __builtin_fma(d0, d0, s0);
      s1 = __builtin_fma(d1, d1, s1);
      s2 = __builtin_fma(d2, d2, s2);
      s3 = __builtin_fma(d3, d3, s3);
    }
  }
  const double s = wave_sum((s0 + s1) + (s2 + s3));
  __shared__ double part[kNormThreads / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = part[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) t += part[w];
    a.partial[(int64_t)p * a.chunks + c] = t;
  }
}

// One wave per slice: lane l adds the partials l + 64 (8 m + k), k = 0..7, into eight sums
// (so that eight loads are in flight, not one chain of dependent adds), m in order, then the
// eight in a fixed tree, then a butterfly.
__global__ __launch_bounds__(64) void state_norms_final_kernel(const NormArgs a) {
  const int p = blockIdx.x;
  const double* part = a.partial + (int64_t)p * a.chunks;
  double t[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int j0 = threadIdx.x; j0 < a.chunks; j0 += 8 * 64) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + 64 * k;
      t[k] += j < a.chunks ? part[j] : 0.0;
    }
  }
  double s = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  s = wave_sum(s);
  if (threadIdx.x == 0) a.norms[p] = (float)sqrt(s);
}

constexpr int kPlanThreads = AS_MAX_PARTITIONS;

// Group error of group k (sum of weights[j] * v[j] over the group, ascending j).
__device__ __forceinline__ float group_sum(const float* wv, int k, int group, int P) {
  const int j1 = (k + 1) * group < P ? (k + 1) * group : P;
  float s = 0.f;
  for (int j = k * group; j < j1; ++j) s += wv[j];
  return s;
}

__global__ __launch_bounds__(kPlanThreads) void planner_decide_kernel(const PlanArgs a) {
  __shared__ float wd[kPlanThreads];
  const int i = threadIdx.x;
  const float drift = a.local_drift[0];
  if (i < a.P) {
    const float alpha = a.anchor_norms[i] / a.anchor_norms[a.local];   // Eq. 9
    const float delta = alpha * drift;                                 // Eq. 10
    if (a.alpha) a.alpha[i] = alpha;
    if (a.delta) a.delta[i] = delta;
    wd[i] = a.weights[i] * delta;
  }
  __syncthreads();
  const int G = (a.P + a.group - 1) / a.group;
  if (i < G) {
    const float e = group_sum(wd, i, a.group, a.P);                    // Eq. 12
    if (a.ase) a.ase[i] = e;
    a.compute[i] = (i == a.local / a.group || e > a.eps[0]) ? 1 : 0;  // Eq. 13
  }
  if (i == 0) a.anchor[0] = drift > a.eps_local ? 1 : 0;              // Algorithm 1
}

__global__ __launch_bounds__(kPlanThreads) void planner_epsilon_kernel(const PlanArgs a) {
  __shared__ float wc[kPlanThreads];
  __shared__ float E[kPlanThreads];
  const int i = threadIdx.x;
  if (i < a.P) wc[i] = a.weights[i] * a.corr_norms[i];
  __syncthreads();
  const int G = (a.P + a.group - 1) / a.group;
  const int lg = a.local / a.group;
  if (i < G) E[i] = group_sum(wc, i, a.group, a.P);
  __syncthreads();
  const int Gp = G - 1;
  int m = (int)floorf(a.reuse_fraction * (float)Gp);
  m = m < 0 ? 0 : (m > Gp ? Gp : m);
  if (m == 0) {
    if (i == 0) a.eps_out[0] = -INFINITY;
    return;
  }
  // rank of group i among the non-local groups (ties broken by index): the one of
  // rank m - 1 is the m-th smallest
  if (i < G && i != lg) {
    int rank = 0;
    for (int k = 0; k < G; ++k)
      if (k != lg && (E[k] < E[i] || (E[k] == E[i] && k < i))) ++rank;
    if (rank == m - 1) a.eps_out[0] = E[i];
  }
}

}  // namespace

hipError_t launch_state_norms(const NormArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.chunks, (unsigned)a.P);
  if (a.b) hipLaunchKernelGGL(state_norms_partial_kernel<true>, grid, dim3(kNormThreads), 0, stream, a);
  else hipLaunchKernelGGL(state_norms_partial_kernel<false>, grid, dim3(kNormThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(state_norms_final_kernel, dim3((unsigned)a.P), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_planner_decide(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(planner_decide_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_planner_epsilon(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(planner_epsilon_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace as
