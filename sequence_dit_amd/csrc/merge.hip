// Composition of n attention states (OUT, LSE) into one, and group-wise composition.
//   DiTango review page (pith.science), axiom ledger, Eq. 1-2: states compose
//   associatively and commutatively (the online-softmax identity); "What carries
//   the argument": several remote partitions are merged into one cached state and
//   folded into the output later; "If this is right": composed states can be
//   merged into coarser groups under memory pressure, a state being about half the
//   size of the KV it summarises.
//
// The kernels are HBM-bound: every byte of every input is read once, every output
// byte written once. One lane owns 4 consecutive elements of one row (16 bytes of
// fp32 OUT), or 8 of a bf16 OUT whose pointers are 16-byte aligned (else 4), so a
// wave reads a contiguous run of 16-byte accesses per input per load instruction. Inputs whose weight is exactly zero (empty states) are neither read
// nor added, and the accumulator starts at -0.0 (the additive identity of IEEE
// arithmetic), so composing any state with empty states returns it bit for bit
// (for fp32 OUT; a bf16 OUT is re-rounded, which is also exact for bf16 inputs).
// Arithmetic is fp32 whatever the storage type; bf16 OUT is written rounded to
// nearest even.
//
// merge_rows_kernel (8 to 64 lanes per row) loads each row's LSE values once and
// shares the weights through LDS; merge_kernel is the general path (any D that is
// a multiple of 4), where every lane of a row reads the row's LSE values. In the
// batched mode (group-wise composition) grid.y is the group and the inputs of a
// group are consecutive slices of one partition-major block.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;

// 4 consecutive OUT elements starting at element `off` of a state, as fp32.
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t off) {
  if (BF16) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const __bf16*>(base) + off));
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                 __uint_as_float(v[1] & 0xffff0000u)};
  }
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off));
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t off, f32x4 r) {
  if (BF16) {
    const bf16x4 h = {(__bf16)r[0], (__bf16)r[1], (__bf16)r[2], (__bf16)r[3]};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), reinterpret_cast<u32x2*>(static_cast<__bf16*>(base) + off));
  } else {
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(static_cast<float*>(base) + off));
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 bf16_pair_to_f32(unsigned lo, unsigned hi) {
  return f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u), __uint_as_float(hi << 16),
               __uint_as_float(hi & 0xffff0000u)};
}

// 4*V consecutive OUT elements at element `off` (V = 2 only for bf16: one 16-byte load).
template <bool BF16, int V>
__device__ __forceinline__ void loadv(const void* base, int64_t off, f32x4 (&x)[V]) {
  if (BF16 && V == 2) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(base) + off));
    x[0] = bf16_pair_to_f32(w[0], w[1]);
    x[V - 1] = bf16_pair_to_f32(w[2], w[3]);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = load4<BF16>(base, off + 4 * v);
  }
}

template <bool BF16, int V>
__device__ __forceinline__ void storev(void* base, int64_t off, const f32x4 (&r)[V]) {
  if (BF16 && V == 2) {
    const bf16x8 h = {(__bf16)r[0][0], (__bf16)r[0][1], (__bf16)r[0][2], (__bf16)r[0][3],
                      (__bf16)r[V - 1][0], (__bf16)r[V - 1][1], (__bf16)r[V - 1][2], (__bf16)r[V - 1][3]};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(static_cast<__bf16*>(base) + off));
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) store4<BF16>(base, off + 4 * v, r[v]);
  }
}

// Where the inputs and outputs of the merge handled by this workgroup live.
template <bool IN_BF16, bool OUT_BF16, bool BATCHED>
struct Io {
  const MergeArgs& a;
  int g;   // group (batched mode)
  int n;   // inputs of this merge
  __device__ __forceinline__ explicit Io(const MergeArgs& a_) : a(a_) {
    g = BATCHED ? (int)blockIdx.y : 0;
    n = BATCHED ? min(a.group, a.n - g * a.group) : a.n;
  }
  __device__ __forceinline__ const float* lse(int k) const {
    return BATCHED ? a.base_lse + (int64_t)(g * a.group + k) * a.rows : a.lses[k];
  }
  __device__ __forceinline__ const void* out(int k) const {
    if (!BATCHED) return a.outs[k];
    const int64_t e = (int64_t)(g * a.group + k) * a.rows * a.D;
    return IN_BF16 ? (const void*)(static_cast<const __bf16*>(a.base_out) + e)
                   : (const void*)(static_cast<const float*>(a.base_out) + e);
  }
  __device__ __forceinline__ void* dst() const {
    const int64_t e = (int64_t)g * a.rows * a.D;
    return OUT_BF16 ? (void*)(static_cast<__bf16*>(a.out) + e) : (void*)(static_cast<float*>(a.out) + e);
  }
  __device__ __forceinline__ float* dst_lse() const { return a.lse + (int64_t)g * a.rows; }
};

template <bool IN_BF16, bool OUT_BF16, bool BATCHED>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeArgs a) {
  const Io<IN_BF16, OUT_BF16, BATCHED> io(a);
  const int cpr = a.D >> 2;  // 4-element chunks per row
  const int64_t total = a.rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * kMergeThreads;
  for (int64_t c = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x; c < total; c += stride) {
    const int64_t row = c / cpr;
    const int col = (int)(c - row * cpr);
    float M = -INFINITY;
    for (int k = 0; k < io.n; ++k) M = fmaxf(M, io.lse(k)[row]);
    const int64_t off = row * a.D + 4 * col;
    if (M == -INFINITY) {  // every input empty: the empty state
      store4<OUT_BF16>(io.dst(), off, f32x4{0.f, 0.f, 0.f, 0.f});
      if (col == 0) io.dst_lse()[row] = -INFINITY;
      continue;
    }
    f32x4 acc = {-0.f, -0.f, -0.f, -0.f};
    float S = 0.f;
    int k = 0;
    for (; k + 4 <= io.n; k += 4) {
      float w[4];
      f32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = expf(io.lse(k + j)[row] - M);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = (w[j] != 0.f) ? load4<IN_BF16>(io.out(k + j), off) : f32x4{0.f, 0.f, 0.f, 0.f};
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
    for (; k < io.n; ++k) {
      const float w = expf(io.lse(k)[row] - M);
      if (w != 0.f) {
        const f32x4 x = load4<IN_BF16>(io.out(k), off);
        S += w;
        acc[0] = __builtin_fmaf(w, x[0], acc[0]);
        acc[1] = __builtin_fmaf(w, x[1], acc[1]);
        acc[2] = __builtin_fmaf(w, x[2], acc[2]);
        acc[3] = __builtin_fmaf(w, x[3], acc[3]);
      }
    }
    store4<OUT_BF16>(io.dst(), off, f32x4{acc[0] / S, acc[1] / S, acc[2] / S, acc[3] / S});
    if (col == 0) io.dst_lse()[row] = M + logf(S);
  }
}


// Fast path for CPR in {8, 16, 32, 64} lanes per row, each lane owning 4*V elements
// (V = 2 for bf16 inputs: one 16-byte load per input): a wave owns 64/CPR rows;
// the n LSE values of a row are loaded once (one per lane of the row group), the
// row's max, weights and their sum are reduced within the group, and the weights
// are handed to the row's lanes through LDS (broadcast reads), so the streaming
// loop issues only the OUT loads, with nontemporal hints (the inputs are read once).
template <int CPR, int V, bool IN_BF16, bool OUT_BF16, bool BATCHED>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_kernel(const MergeArgs a) {
  constexpr int RPW = 64 / CPR;                 // rows per wave
  constexpr int RPB = RPW * (kMergeThreads / 64);
  constexpr int E = 4 * V;                      // elements per lane
  __shared__ float wsh[kMergeThreads / 64][RPW][AS_MAX_MERGE];
  const Io<IN_BF16, OUT_BF16, BATCHED> io(a);
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
    Lv[u] = (live && k < io.n) ? io.lse(k)[row] : -INFINITY;
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
  const int64_t off = row * a.D + E * j;
  f32x4 acc[V];
  if (empty) {
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    storev<OUT_BF16, V>(io.dst(), off, acc);
    if (j == 0) io.dst_lse()[row] = -INFINITY;
    return;
  }
  // 2. stream the inputs with non-zero weight
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = f32x4{-0.f, -0.f, -0.f, -0.f};
  int k = 0;
  for (; k + 4 <= io.n; k += 4) {
    float w[4];
    f32x4 x[4][V];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = wsh[wave][g][k + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (w[u] != 0.f) loadv<IN_BF16, V>(io.out(k + u), off, x[u]);
      else {
#pragma unroll
        for (int v = 0; v < V; ++v) x[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (w[u] != 0.f) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[v][e] = __builtin_fmaf(w[u], x[u][v][e], acc[v][e]);
      }
  }
  for (; k < io.n; ++k) {
    const float w = wsh[wave][g][k];
    if (w != 0.f) {
      f32x4 x[V];
      loadv<IN_BF16, V>(io.out(k), off, x);
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[v][e] = __builtin_fmaf(w, x[v][e], acc[v][e]);
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = f32x4{acc[v][0] / S, acc[v][1] / S, acc[v][2] / S, acc[v][3] / S};
  storev<OUT_BF16, V>(io.dst(), off, acc);
  if (j == 0) io.dst_lse()[row] = M + logf(S);
}

template <int V, bool IN_BF16, bool OUT_BF16, bool BATCHED>
bool launch_rows(const MergeArgs& a, unsigned groups, hipStream_t stream) {
  const int cpr = a.D / (4 * V);
  if (a.D % (4 * V) || (cpr != 8 && cpr != 16 && cpr != 32 && cpr != 64)) return false;
  const int64_t rpb = (64 / cpr) * (kMergeThreads / 64);
  const dim3 grid((unsigned)((a.rows + rpb - 1) / rpb), groups), block(kMergeThreads);
  switch (cpr) {
    case 8: hipLaunchKernelGGL((merge_rows_kernel<8, V, IN_BF16, OUT_BF16, BATCHED>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((merge_rows_kernel<16, V, IN_BF16, OUT_BF16, BATCHED>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((merge_rows_kernel<32, V, IN_BF16, OUT_BF16, BATCHED>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_rows_kernel<64, V, IN_BF16, OUT_BF16, BATCHED>), grid, block, 0, stream, a); break;
  }
  return true;
}

template <bool IN_BF16, bool OUT_BF16, bool BATCHED>
hipError_t launch(const MergeArgs& a, hipStream_t stream) {
  const unsigned groups = BATCHED ? (unsigned)((a.n + a.group - 1) / a.group) : 1u;
  // bf16 inputs whose rows and pointers allow it: 8 elements (16 bytes) per lane
  if constexpr (IN_BF16) {
    if (a.vec2 && launch_rows<2, IN_BF16, OUT_BF16, BATCHED>(a, groups, stream)) return hipGetLastError();
  }
  if (launch_rows<1, IN_BF16, OUT_BF16, BATCHED>(a, groups, stream)) return hipGetLastError();
  const int cpr = a.D / 4;
  const int64_t total = a.rows * cpr;
  int64_t blocks = (total + kMergeThreads - 1) / kMergeThreads;
  if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;  // grid-stride beyond this
  hipLaunchKernelGGL((merge_kernel<IN_BF16, OUT_BF16, BATCHED>), dim3((unsigned)blocks, groups), dim3(kMergeThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool BATCHED>
hipError_t dispatch(const MergeArgs& a, hipStream_t stream) {
  if (a.in_bf16) return a.out_bf16 ? launch<true, true, BATCHED>(a, stream) : launch<true, false, BATCHED>(a, stream);
  return a.out_bf16 ? launch<false, true, BATCHED>(a, stream) : launch<false, false, BATCHED>(a, stream);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.rows * (a.D / 4) <= 0) return hipSuccess;
  return a.group > 0 ? dispatch<true>(a, stream) : dispatch<false>(a, stream);
}

}  // namespace as
