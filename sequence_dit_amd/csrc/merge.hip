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
// wave reads a contiguous run of 16-byte accesses per input per load instruction. Inputs
// whose weight is exactly zero (empty states) are not added (nor read, but for the first
// four fp8 inputs of a row), and the accumulator starts at -0.0 (the additive identity of IEEE
// arithmetic), so composing any state with empty states returns it bit for bit
// (for fp32 OUT; a bf16 OUT is re-rounded, which is also exact for bf16 inputs).
// Arithmetic is fp32 whatever the storage type; bf16 OUT is written rounded to
// nearest even. An fp8 state (a payload of E4M3 codes with one float32 factor per row)
// is read by folding its row's factor into the row's weight; an fp8 OUT is written as
// the codes of OUT * (448 / amax), rounded to nearest even, with the factor amax / 448,
// amax being the row's largest |OUT| (FastUSP page, abstract: FP8-quantised attention
// traffic).
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

// 4 consecutive OUT elements starting at element `off` of a state, as fp32 (fp32 or
// bf16 storage).
template <int IN>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t off) {
  static_assert(IN != kOutFP8, "fp8 states are read by loadv");
  if (IN == kOutBF16) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const __bf16*>(base) + off));
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
                 __uint_as_float(v[1] & 0xffff0000u)};
  }
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off));
}

template <int OUT>
__device__ __forceinline__ void store4(void* base, int64_t off, f32x4 r) {
  static_assert(OUT != kOutFP8, "fp8 states are written by store_fp8_row");
  if (OUT == kOutBF16) {
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

// 4 E4M3 codes (one 32-bit word, lowest address first) as fp32 values, exactly.
__device__ __forceinline__ f32x4 fp8x4_to_f32(unsigned w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 4*V E4M3 codes at element (= byte) `off`, as V words, in one load.
template <int V>
__device__ __forceinline__ void load_codes(const void* base, int64_t off, unsigned (&r)[V]) {
  const unsigned char* p8 = static_cast<const unsigned char*>(base) + off;
  if constexpr (V == 4) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p8));
#pragma unroll
    for (int v = 0; v < 4; ++v) r[v] = w[v];
  } else if constexpr (V == 2) {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p8));
    r[0] = w[0];
    r[V - 1] = w[1];
  } else {
    static_assert(V == 1, "4, 8 or 16 codes per load");
    r[0] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p8));
  }
}

// 4*V consecutive OUT elements at element `off` of fp32 or bf16 storage (V = 2 for bf16:
// one 16-byte load; fp8 codes are read by load_codes).
template <int IN, int V>
__device__ __forceinline__ void loadv(const void* base, int64_t off, f32x4 (&x)[V]) {
  static_assert(IN != kOutFP8, "fp8 codes are read by load_codes");
  if (IN == kOutBF16 && V == 2) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(base) + off));
    x[0] = bf16_pair_to_f32(w[0], w[1]);
    x[V - 1] = bf16_pair_to_f32(w[2], w[3]);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) x[v] = load4<IN>(base, off + 4 * v);
  }
}

template <int OUT, int V>
__device__ __forceinline__ void storev(void* base, int64_t off, const f32x4 (&r)[V]) {
  if (OUT == kOutBF16 && V == 2) {
    const bf16x8 h = {(__bf16)r[0][0], (__bf16)r[0][1], (__bf16)r[0][2], (__bf16)r[0][3],
                      (__bf16)r[V - 1][0], (__bf16)r[V - 1][1], (__bf16)r[V - 1][2], (__bf16)r[V - 1][3]};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(static_cast<__bf16*>(base) + off));
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) store4<OUT>(base, off + 4 * v, r[v]);
  }
}

// Four values as E4M3 codes (one 32-bit word, lowest address first), rounded to nearest
// even, after clamping to the largest finite code (448).
__device__ __forceinline__ unsigned f32x4_to_fp8(f32x4 x) {
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = fminf(fmaxf(x[e], -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (unsigned)w;
}

// Where the inputs and outputs of the merge handled by this workgroup live.
template <int IN, int OUT, bool BATCHED>
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
    const int64_t s = g * a.group + k;   // slice of the block
    if (IN == kOutFP8) return static_cast<const char*>(a.base_out) + s * a.payload_bytes;
    const int64_t e = s * a.rows * a.D;
    return IN == kOutBF16 ? (const void*)(static_cast<const __bf16*>(a.base_out) + e)
                          : (const void*)(static_cast<const float*>(a.base_out) + e);
  }
  // fp8 inputs: the row factors of input k
  __device__ __forceinline__ const float* in_factor(int k) const {
    return reinterpret_cast<const float*>(static_cast<const char*>(out(k)) + a.rows * a.D);
  }
  __device__ __forceinline__ void* dst() const {
    if (OUT == kOutFP8) return static_cast<char*>(a.out) + (int64_t)g * a.payload_bytes;
    const int64_t e = (int64_t)g * a.rows * a.D;
    return OUT == kOutBF16 ? (void*)(static_cast<__bf16*>(a.out) + e) : (void*)(static_cast<float*>(a.out) + e);
  }
  __device__ __forceinline__ float* dst_factor() const {
    return reinterpret_cast<float*>(static_cast<char*>(dst()) + a.rows * a.D);
  }
  __device__ __forceinline__ float* dst_lse() const { return a.lse + (int64_t)g * a.rows; }
};

template <int IN, int OUT, bool BATCHED>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeArgs a) {
  const Io<IN, OUT, BATCHED> io(a);
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
      store4<OUT>(io.dst(), off, f32x4{0.f, 0.f, 0.f, 0.f});
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
      for (int j = 0; j < 4; ++j) x[j] = (w[j] != 0.f) ? load4<IN>(io.out(k + j), off) : f32x4{0.f, 0.f, 0.f, 0.f};
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
        const f32x4 x = load4<IN>(io.out(k), off);
        S += w;
        acc[0] = __builtin_fmaf(w, x[0], acc[0]);
        acc[1] = __builtin_fmaf(w, x[1], acc[1]);
        acc[2] = __builtin_fmaf(w, x[2], acc[2]);
        acc[3] = __builtin_fmaf(w, x[3], acc[3]);
      }
    }
    store4<OUT>(io.dst(), off, f32x4{acc[0] / S, acc[1] / S, acc[2] / S, acc[3] / S});
    if (col == 0) io.dst_lse()[row] = M + logf(S);
  }
}


// An fp8 OUT row: lane j of the row's CPR lanes holds the 4V values at element `off`;
// amax is the row's largest |value| (0 for a zero row: codes 0, factor 0).
template <int CPR, int V, typename IO>
__device__ __forceinline__ void store_fp8_row(const IO& io, int64_t row, int64_t off, int j, const f32x4 (&x)[V],
                                              float amax) {
  const float qf = amax > 0.f ? 448.0f / amax : 0.f;
  unsigned c[V];
#pragma unroll
  for (int v = 0; v < V; ++v) c[v] = f32x4_to_fp8(f32x4{x[v][0] * qf, x[v][1] * qf, x[v][2] * qf, x[v][3] * qf});
  unsigned char* p8 = static_cast<unsigned char*>(io.dst()) + off;
  if constexpr (V == 4) __builtin_nontemporal_store(u32x4{c[0], c[1], c[2], c[3]}, reinterpret_cast<u32x4*>(p8));
  else if constexpr (V == 2) __builtin_nontemporal_store(u32x2{c[0], c[1]}, reinterpret_cast<u32x2*>(p8));
  else __builtin_nontemporal_store(c[0], reinterpret_cast<unsigned*>(p8));
  if (j == 0) io.dst_factor()[row] = amax / 448.0f;
}

// Fast path for CPR in {8, 16, 32, 64} lanes per row, each lane owning 4*V elements
// (V = 2 for bf16 inputs: one 16-byte load per input): a wave owns 64/CPR rows;
// the n LSE values of a row are loaded once (one per lane of the row group), the
// row's max, weights and their sum are reduced within the group, and the weights
// are handed to the row's lanes through LDS (broadcast reads), so the streaming
// loop issues only the OUT loads, with nontemporal hints (the inputs are read once).
// Inputs whose weight is zero are not read, except the first four fp8 inputs of a row, whose
// codes are loaded before the weights (and still not added).
// fp8 states go through this path only (fp8 inputs: V = D / 32 up to 4, 4 to 16 codes per
// lane; an fp8 OUT takes the lanes of its input's storage).
template <int CPR, int V, int IN, int OUT, bool BATCHED>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_kernel(const MergeArgs a) {
  constexpr int RPW = 64 / CPR;                 // rows per wave
  constexpr int RPB = RPW * (kMergeThreads / 64);
  constexpr int E = 4 * V;                      // elements per lane
  __shared__ float wsh[kMergeThreads / 64][RPW][AS_MAX_MERGE];
  const Io<IN, OUT, BATCHED> io(a);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / CPR, j = lane % CPR;     // row within the wave, lane within the row
  const int64_t row = (int64_t)blockIdx.x * RPB + wave * RPW + g;
  const bool live = row < a.rows;
  // 1. LSE of inputs j, j + CPR, ... of this row (and an fp8 input's row factor, loaded
  // alongside, not after the weight); max over the row group
  constexpr int NU = AS_MAX_MERGE / CPR > 0 ? AS_MAX_MERGE / CPR : 1;
  const int64_t off = row * a.D + E * j;
  // 0. fp8 inputs: the codes of the first 4 inputs, loaded before their weights are known
  // (not added when the weight is zero), so that their latency overlaps step 1's
  constexpr int U8 = 4;
  unsigned r8[IN == kOutFP8 ? U8 : 1][V];
  if constexpr (IN == kOutFP8) {
#pragma unroll
    for (int u = 0; u < U8; ++u)
      if (live && u < io.n) load_codes<V>(io.out(u), off, r8[u]);
  }
  float Lv[NU], Fv[NU];
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < AS_MAX_MERGE / CPR; ++u) {
    const int k = j + u * CPR;
    Lv[u] = (live && k < io.n) ? io.lse(k)[row] : -INFINITY;
    if constexpr (IN == kOutFP8) Fv[u] = (live && k < io.n) ? io.in_factor(k)[row] : 0.f;
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
    // an fp8 input's row factor scales its codes: folded into the weight of its OUT
    float wf = w;
    if constexpr (IN == kOutFP8) wf = w * Fv[u];
    if (k < AS_MAX_MERGE) wsh[wave][g][k] = wf;
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) S += __shfl_xor(S, m, CPR);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // (a row past the end is empty: its lanes leave here, all of a row group together)
  if (!live) return;
  f32x4 acc[V];
  if (empty) {   // (an fp8 OUT: codes 0 and factor 0)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (OUT == kOutFP8) store_fp8_row<CPR, V>(io, row, off, j, acc, 0.f);
    else storev<OUT, V>(io.dst(), off, acc);
    if (j == 0) io.dst_lse()[row] = -INFINITY;
    return;
  }
  // 2. stream the inputs with non-zero weight, in input order
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = f32x4{-0.f, -0.f, -0.f, -0.f};
  int k = 0;
  if constexpr (IN == kOutFP8) {
    // fp8 inputs, 4 at a time: the codes of the next 4 are loaded before the current 4 are
    // widened and added (raw code words: V registers per input)
    for (; k < io.n; k += U8) {
      unsigned nx[U8][V];
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int kk = k + U8 + u;
        if (kk < io.n && wsh[wave][g][kk] != 0.f) load_codes<V>(io.out(kk), off, nx[u]);
        else {
#pragma unroll
          for (int v = 0; v < V; ++v) nx[u][v] = 0u;
        }
      }
#pragma unroll
      for (int u = 0; u < U8; ++u) {
        const int kk = k + u;
        const float w = kk < io.n ? wsh[wave][g][kk] : 0.f;
        if (w != 0.f) {
#pragma unroll
          for (int v = 0; v < V; ++v) {
            const f32x4 x = fp8x4_to_f32(r8[u][v]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[v][e] = __builtin_fmaf(w, x[e], acc[v][e]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U8; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v) r8[u][v] = nx[u][v];
    }
  } else {
    for (; k + 4 <= io.n; k += 4) {
      float w[4];
      f32x4 x[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = wsh[wave][g][k + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (w[u] != 0.f) loadv<IN, V>(io.out(k + u), off, x[u]);
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
        loadv<IN, V>(io.out(k), off, x);
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[v][e] = __builtin_fmaf(w, x[v][e], acc[v][e]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = f32x4{acc[v][0] / S, acc[v][1] / S, acc[v][2] / S, acc[v][3] / S};
  if constexpr (OUT == kOutFP8) {
    float mx = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(acc[v][e]));
    // the row's CPR lanes hold its D values (and are all here: liveness is per row)
#pragma unroll
    for (int m = CPR / 2; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, CPR));
    store_fp8_row<CPR, V>(io, row, off, j, acc, mx);
  } else {
    storev<OUT, V>(io.dst(), off, acc);
  }
  if (j == 0) io.dst_lse()[row] = M + logf(S);
}

template <int V, int IN, int OUT, bool BATCHED>
bool launch_rows(const MergeArgs& a, unsigned groups, hipStream_t stream) {
  const int cpr = a.D / (4 * V);
  if (a.D % (4 * V) || (cpr != 8 && cpr != 16 && cpr != 32 && cpr != 64)) return false;
  const int64_t rpb = (64 / cpr) * (kMergeThreads / 64);
  const dim3 grid((unsigned)((a.rows + rpb - 1) / rpb), groups), block(kMergeThreads);
  switch (cpr) {
    case 8: hipLaunchKernelGGL((merge_rows_kernel<8, V, IN, OUT, BATCHED>), grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL((merge_rows_kernel<16, V, IN, OUT, BATCHED>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((merge_rows_kernel<32, V, IN, OUT, BATCHED>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_rows_kernel<64, V, IN, OUT, BATCHED>), grid, block, 0, stream, a); break;
  }
  return true;
}

template <int IN, int OUT, bool BATCHED>
hipError_t launch(const MergeArgs& a, hipStream_t stream) {
  const unsigned groups = BATCHED ? (unsigned)((a.n + a.group - 1) / a.group) : 1u;
  // The lanes per row (and so the order of the row's LSE reductions) follow the input's
  // storage alone: the same inputs give the same LSE and the same fp32 OUT whatever the
  // output's storage, so an fp8 OUT holds the codes of that fp32 OUT.
  if constexpr (IN == kOutFP8) {
    // fp8 inputs: D in {32, 64, 128, 256} (checked by the caller), 4 * min(D / 32, 4) codes
    // per lane: one 4-, 8- or 16-byte load per input
    if (a.D == 32 && launch_rows<1, IN, OUT, BATCHED>(a, groups, stream)) return hipGetLastError();
    if (a.D == 64 && launch_rows<2, IN, OUT, BATCHED>(a, groups, stream)) return hipGetLastError();
    if ((a.D == 128 || a.D == 256) && launch_rows<4, IN, OUT, BATCHED>(a, groups, stream)) return hipGetLastError();
    return hipErrorInvalidValue;
  } else {
    // bf16 inputs whose rows and pointers allow it: 8 elements (16 bytes) per lane
    if constexpr (IN == kOutBF16) {
      if (a.vec2 && launch_rows<2, IN, OUT, BATCHED>(a, groups, stream)) return hipGetLastError();
    }
    if (launch_rows<1, IN, OUT, BATCHED>(a, groups, stream)) return hipGetLastError();
    if constexpr (OUT == kOutFP8) {
      return hipErrorInvalidValue;   // (D in {32, 64, 128, 256}: a row path above took it)
    } else {
      const int cpr = a.D / 4;
      const int64_t total = a.rows * cpr;
      int64_t blocks = (total + kMergeThreads - 1) / kMergeThreads;
      if (blocks > (int64_t)1 << 20) blocks = (int64_t)1 << 20;  // grid-stride beyond this
      hipLaunchKernelGGL((merge_kernel<IN, OUT, BATCHED>), dim3((unsigned)blocks, groups), dim3(kMergeThreads), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
}

template <int IN, bool BATCHED>
hipError_t dispatch_out(const MergeArgs& a, hipStream_t stream) {
  switch (a.out_kind) {
    case kOutF32: return launch<IN, kOutF32, BATCHED>(a, stream);
    case kOutBF16: return launch<IN, kOutBF16, BATCHED>(a, stream);
    case kOutFP8: return launch<IN, kOutFP8, BATCHED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BATCHED>
hipError_t dispatch(const MergeArgs& a, hipStream_t stream) {
  switch (a.in_kind) {
    case kOutF32: return dispatch_out<kOutF32, BATCHED>(a, stream);
    case kOutBF16: return dispatch_out<kOutBF16, BATCHED>(a, stream);
    case kOutFP8: return dispatch_out<kOutFP8, BATCHED>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.rows * (a.D / 4) <= 0) return hipSuccess;
  return a.group > 0 ? dispatch<true>(a, stream) : dispatch<false>(a, stream);
}

}  // namespace as
