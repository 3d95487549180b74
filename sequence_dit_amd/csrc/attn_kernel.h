// Template of the MFMA partition-attention kernel shared by the sources that instantiate it
// (partition_attn.hip: bf16 inputs; partition_attn_fp8.hip: fp8 E4M3 queries and keys;
// partition_attn_grouped.hip: grouped launches that compose the states of consecutive
// partitions in the epilogue). Internal header; its contents live in an anonymous namespace,
// so every including source gets its own copies of what it instantiates.
//
// Partition attention on CDNA4 (gfx950): per query row and per KV partition i,
// the attention state AS(i) = (OUT(i), LSE(i)) of exact softmax attention
// restricted to the keys of partition i.
//   DiTango review page (pith.science), "What carries the argument": the state of a
//   partition is its partial attention output with the log-sum-exp of its scores.
//
// bf16 kernel design (one workgroup = 8 waves = 256 query rows x one (batch, head)
// x one partition; one wave = 32 query rows; two waves per SIMD; key tiles of 64
// keys at D = 128 and 128 at D = 64):
//   * The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (M = 32 keys, N = 32 queries, K = 16 of D). In that accumulator layout a lane
//     holds 16 keys of ONE query row, so the row max needs one cross-half swap
//     (v_permlane32_swap) and the row sum stays lane-local until the epilogue.
//   * The accumulator registers of S^T are, key for key, the B operand of
//     O^T = V^T P^T (M = 32 of D, N = 32 queries, K = 16 keys) once rounded to bf16:
//     P never leaves registers.
//   * Q stays in registers for the whole partition. K tiles are staged in LDS as
//     [key][d] rows padded to 2D + 16 bytes; V tiles are transposed in registers on
//     their way into LDS ([d][key] rows of a tile's keys padded by 16 bytes, 4-key groups
//     placed so that one 16-byte read per lane is the V^T operand). The padding makes
//     the 16-byte operand reads conflict-free. Two slots per operand: the global
//     loads of a tile are issued one tile ahead of its LDS store.
//   * The 8 waves form two groups that alternate an MFMA phase with a softmax phase,
//     one phase apart, so that on every SIMD one wave's softmax runs beside the
//     other's MFMAs; each wave's code stays a plain sequence of phases.
//   * Online softmax in the exp2 domain with a lazy rescale: the running max is
//     only moved (and O, l rescaled) when a new score exceeds it by more than
//     2^64, which is exact because the same max is used for O and l.
//   * Workgroups sharing a (batch, head, partition) are mapped to the same XCD so
//     that its L2 serves their common K/V tiles.
//
// fp8 queries and keys (template flag QK8): Q and K are FP8 E4M3 codes and
// S^T = K Q^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales), 2 D/64
// steps per tile of 32 bytes of K per lane; K rows in LDS are D + 16 bytes. The
// per-(batch, head) dequantisation factors fold into the softmax scale. Softmax,
// P, V and PV are the bf16 path's.
//   DiTango review page, reference list: SageAttention (8-bit attention for
//   inference); FastUSP page, prior work: the FP8 formats paper (E4M3).
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <type_traits>
#include <functional>
#include <vector>

#include "as_internal.h"

namespace as {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Stores of OUT elements: fp32, or bf16 rounded to nearest even (fp8 payloads have their
// own epilogue).
template <int OUT>
__device__ __forceinline__ void store_out4(void* base, int64_t off, f32x4 v) {
  if (OUT == kOutBF16) {
    const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(base) + off) = __builtin_bit_cast(u32x2, h);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = v;
  }
}

template <int OUT>
__device__ __forceinline__ void store_out1(void* base, int64_t off, float v) {
  if (OUT == kOutBF16) static_cast<__bf16*>(base)[off] = (__bf16)v;
  else static_cast<float*>(base)[off] = v;
}

// Four values as E4M3 codes (one 32-bit word, lowest address first), rounded to nearest
// even; callers keep |x| <= 448.
__device__ __forceinline__ unsigned fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}
__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

#ifdef AS_WG_STAMPS
// Diagnostics build only (compiled with -DAS_WG_STAMPS into libas_attn_stamps.so, never into
// the product library): workgroup i < kStampWGs of a single-partition launch records, from
// its first thread, 8 words: s_memrealtime (100 MHz) at its start, after its first barrier
// (K tile 0 in LDS), after its last tile and at its end; s_memtime (shader clock) at its
// start and end; its query tile and partition; its HW_ID and XCC_ID registers.
constexpr int kStampWGs = 16384;
__device__ unsigned long long as_wg_stamps[kStampWGs * 8];
#define AS_STAMP(i, value)                                                                     \
  do {                                                                                         \
    if (threadIdx.x == 0 && blockIdx.x < kStampWGs) as_wg_stamps[8 * blockIdx.x + (i)] = (value); \
  } while (0)
#else
#define AS_STAMP(i, value) \
  do {                     \
  } while (0)
#endif

constexpr int kWaves = 8;
constexpr int kQB = 1;                       // 32-row query blocks per wave
constexpr int kRowsPerWave = 32 * kQB;       // 32
constexpr int kBQ = kWaves * kRowsPerWave;   // 256 query rows per workgroup
// Keys per tile: 64 at D = 128. At D = 64 a tile's MFMA work halves while its
// softmax work does not, so the softmax phase is the longer one and every phase
// pays its start, drain and barrier for half the work; a 128-key tile (the
// registers allow twice the S and P of a 64-key one there) halves those costs.
template <int D>
struct Tile {
  static constexpr int KB = D == 64 ? 128 : 64;   // keys per tile
  static constexpr int NKB = KB / 32;             // 32-key MFMA blocks per tile
};
constexpr int kThreads = kWaves * 64;
// Probabilities of a tile may reach 2^64 before the running max is moved (the sum of a
// lane's 32 or 64 of them then stays far inside fp32, and so do O and l).
constexpr float kRescaleLimit = 18446744073709551616.0f;   // 2^64

__device__ __forceinline__ float wave_max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS-only workgroup barrier: waits for this wave's LDS operations, not for its
// outstanding global loads (those are consumed phases later).
// The scheduling fences keep the compiler from moving ALU work of one phase across
// the barrier into the next phase.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// Operand reads in flight during an MFMA phase (one ds_read_b128 per MFMA).
constexpr int kLookahead = 6;


// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Step plan of an fp8 MFMA phase: NS S steps (two 16-byte operand units each) and
// NPV PV steps (one unit each); one S step precedes every R PV steps.
template <int NS_, int NPV_>
struct Fp8Plan {
  static constexpr int NS = NS_, NPV = NPV_, N = NS + NPV, NU = 2 * NS + NPV;
  static constexpr int R = (NS > 0 && NPV > 0) ? NPV / NS : 0;
  static_assert(NS == 0 || NPV == 0 || NPV % NS == 0, "step interleave");
  static constexpr int LA = NU < kLookahead ? NU : kLookahead;
  static constexpr bool is_s(int j) { return NS == 0 ? false : NPV == 0 ? true : j % (R + 1) == 0; }
  static constexpr int idx(int j) {
    return (NS == 0 || NPV == 0) ? j : (j % (R + 1) == 0 ? j / (R + 1) : j - j / (R + 1) - 1);
  }
  static constexpr int ustart(int j) {
    int u = 0;
    for (int i = 0; i < j; ++i) u += is_s(i) ? 2 : 1;
    return u;
  }
  static constexpr int unit_step(int u) {
    int j = 0;
    while (ustart(j + 1) <= u) ++j;
    return j;
  }
};

// LDS layout of one workgroup (bytes). Rows are padded by 16 bytes instead of
// XOR-swizzled, so every operand address is a per-lane base plus a compile-time
// immediate. K tiles are [key][d]; V tiles are transposed, [d][key], with the keys
// of a row permuted so that the 8 keys one lane feeds to an MFMA are contiguous.
template <int D, bool QK8>
struct Lds {
  static constexpr int KP = D * (QK8 ? 1 : 2) + 16;   // K row pitch (fp8 or bf16 keys)
  static constexpr int KTILE = Tile<D>::KB * KP;
  static constexpr int VP = Tile<D>::KB * 2 + 16;   // V^T row pitch
  static constexpr int VTILE = D * VP;
  static constexpr int V0 = 2 * KTILE;         // two K slots, then two V slots
  static constexpr int BYTES = 2 * KTILE + 2 * VTILE;
};

// Position (bytes) of 4-key group g (keys 4g..4g+3 of a tile) in a V^T row.
// The MFMA operand of lane half h for (key block kb, step c) is the key groups
// 8kb+4c+h and 8kb+4c+h+2, stored side by side as 16-byte chunk 4kb+2c+h.
__device__ __forceinline__ constexpr int vt_group_pos(int g) {
  return 16 * (((g >> 2) << 1) | (g & 1)) + 8 * ((g >> 1) & 1);
}

// Q fragments (B operand of S^T) of one lane. bf16: Q[row l32][d = 16ds + 8half .. +7].
// fp8: Q[row l32][d = 64ds + 32half .. +31]; the fp8 MFMA pairs byte j of a lane half
// of A with byte j of the same lane half of B, so K and Q only need the same d order.
template <int D, bool QK8> struct QFrag { bf16x8 v[D / 16]; };
template <int D> struct QFrag<D, true> { i32x8 v[D / 64]; };

// Per-wave state of the bf16 kernel; one wave owns 32 query rows. GR: grouped launch
// (the states of several partitions are composed in the wave's registers, and the row
// sum of the current partition is kept beside the composed one).
template <int D, bool QK8, bool GR = false>
struct Wave {
  static constexpr int NDS = QK8 ? D / 64 : D / 16;   // MFMA k-steps of S^T = K Q^T
  static constexpr int NDB = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int KB = Tile<D>::KB, NKB = Tile<D>::NKB;
  QFrag<D, QK8> qf;      // Q, for the whole partition
  f32x16 s[NKB];         // S^T of the current tile: [kb], reg r <-> key 32kb + 8(r/4) + 4half + r%4
  bf16x8 pf[NKB][2];     // P of the previous tile, B operand of O^T: [kb][c]
  f32x16 o[NDB];         // O^T: [db], reg r <-> d = 32db + 8(r/4) + 4half + r%4
  float m, l;            // running max (log2 domain, scaled) and row sum
  float lp;              // grouped launches: row sum of the current partition (same max as l)
  int k_rd, v_rd;        // LDS read bases of this lane

  // MFMA phase of tile t: S_t = K_t Q^T from K slot KS (if DO_S) and
  // O^T += V_{t-1}^T P_{t-1}^T from V slot VS (if DO_PV). S and PV steps alternate;
  // the operand of step j + LA is read right after the MFMA of step j is issued, and
  // a scheduling fence after every step pins that order, so that LA reads are always
  // in flight (left to itself the scheduler moves a read next to its consumer and
  // the wave drains the LDS queue).
  template <int KS, int VS, bool DO_S, bool DO_PV>
  __device__ __forceinline__ void mfma_phase(const char* smem) {
    if constexpr (QK8) mfma_phase_fp8<KS, VS, DO_S, DO_PV>(smem);
    else mfma_phase_bf16<KS, VS, DO_S, DO_PV>(smem);
  }

  template <int KS, int VS, bool DO_S, bool DO_PV>
  __device__ __forceinline__ void mfma_phase_bf16(const char* smem) {
    using L = Lds<D, QK8>;
    constexpr int NS = DO_S ? NKB * NDS : 0;
    constexpr int NPV = DO_PV ? 2 * NKB * NDB : 0;
    constexpr int N = NS + NPV;
    constexpr int NM = NS < NPV ? NS : NPV;
    constexpr int LA = N < kLookahead ? N : kLookahead;
    const char* kb_ = smem + k_rd + KS * L::KTILE;
    const char* vb_ = smem + v_rd + VS * L::VTILE;
    auto is_s = [](int j) { return NS == 0 ? false : NPV == 0 ? true : (j < 2 * NM ? (j & 1) == 0 : NS > NPV); };
    auto idx = [](int j) { return j < 2 * NM ? j / 2 : j - NM; };
    bf16x8 fr[N > 0 ? N : 1];
    auto load = [&](int j) {
      const int i = idx(j);
      if (is_s(j)) {
        const int ds = i / NKB, kb = i % NKB;
        fr[j] = *reinterpret_cast<const bf16x8*>(kb_ + kb * 32 * L::KP + ds * 32);
      } else {
        const int kbc = i / NDB, db = i % NDB;     // kbc = 2kb + c
        fr[j] = *reinterpret_cast<const bf16x8*>(vb_ + db * 32 * L::VP + 32 * kbc);
      }
    };
    if (DO_S) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    }
#pragma unroll
    for (int j = 0; j < LA; ++j) load(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = idx(j);
      if (is_s(j)) {
        const int ds = i / NKB, kb = i % NKB;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], qf.v[ds], s[kb], 0, 0, 0);
      } else {
        const int kbc = i / NDB, db = i % NDB;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j], pf[kbc >> 1][kbc & 1], o[db], 0, 0, 0);
      }
      if (j + LA < N) load(j + LA);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // fp8 MFMA phase: S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands,
  // unit block scales; 2 * D / 64 steps of 64 d, each reading 32 bytes of K per lane,
  // twice the work of a bf16 step), and the bf16 O^T += V^T P^T steps as above. One
  // S step precedes every R = NPV / NS PV steps. Operand reads go in 16-byte units,
  // kLookahead units ahead, pinned by a scheduling fence after every step.
  template <int KS, int VS, bool DO_S, bool DO_PV>
  __device__ __forceinline__ void mfma_phase_fp8(const char* smem) {
    using L = Lds<D, QK8>;
    using Pl = Fp8Plan<DO_S ? NKB * NDS : 0, DO_PV ? 2 * NKB * NDB : 0>;
    const char* kb_ = smem + k_rd + KS * L::KTILE;
    const char* vb_ = smem + v_rd + VS * L::VTILE;
    i32x8 sf[Pl::NS > 0 ? Pl::NS : 1];
    bf16x8 vf[Pl::NPV > 0 ? Pl::NPV : 1];
    auto load_unit = [&](auto U) {
      constexpr int u = decltype(U)::value;
      if constexpr (u < Pl::NU) {
        constexpr int j = Pl::unit_step(u);
        constexpr int i = Pl::idx(j);
        if constexpr (Pl::is_s(j)) {
          constexpr int h = u - Pl::ustart(j), ds = i / NKB, kb = i % NKB;
          const u32x4 x = *reinterpret_cast<const u32x4*>(kb_ + kb * 32 * L::KP + ds * 64 + 16 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) sf[i][4 * h + e] = (int)x[e];
        } else {
          constexpr int kbc = i / NDB, db = i % NDB;
          vf[i] = *reinterpret_cast<const bf16x8*>(vb_ + db * 32 * L::VP + 32 * kbc);
        }
      }
    };
    if (DO_S) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    }
    static_for<0, Pl::LA>(load_unit);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, Pl::N>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int i = Pl::idx(j);
      if constexpr (Pl::is_s(j)) {
        constexpr int ds = i / NKB, kb = i % NKB;
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sf[i], qf.v[ds], s[kb], 0, 0, 0, 127, 0, 127);
      } else {
        constexpr int kbc = i / NDB, db = i % NDB;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[kbc >> 1][kbc & 1], o[db], 0, 0, 0);
      }
      static_for<Pl::ustart(j) + Pl::LA, Pl::ustart(j + 1) + Pl::LA>(load_unit);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // Softmax phase of tile t: online softmax of S_t (exp2 domain, lazy rescale) -> P_t.
  // valid = keys of the tile inside the partition.
  // FIRST: the row's first tile (of the partition, or of the group in grouped launches).
  template <bool FIRST>
  __device__ __forceinline__ void softmax_phase(int valid, float c2, int half) {
    if constexpr (GR) {
      // Grouped launches meet masked tiles inside the tile loop (at every partition end):
      // one copy of the softmax body with the mask block in front keeps the loop's register
      // assignment the same on both paths (two inlined copies make the allocator shuffle
      // the accumulators between them).
      if (valid < KB) {
        mask_tail(valid, c2, half);
        c2 = 1.0f;
      }
      softmax<false, FIRST>(valid, c2, half);
    } else {
      // single partition: the masked tile is the last one, outside the steady-state loop
      if (valid < KB) softmax<true, FIRST>(valid, c2, half);
      else softmax<false, FIRST>(valid, c2, half);
    }
  }

  // Keys at or past `valid` of the tile: scores scaled by c2, masked ones set to -inf.
  // Single-partition launches: a 32-key block wholly inside or wholly past the end (a
  // wave-uniform test) is scaled or cleared without a comparison per key. (Grouped launches
  // mask inside the tile loop, where the three-way branch costs more than it saves.)
  __device__ __forceinline__ void mask_tail(int valid, float c2, int half) {
    const int lim = valid - 4 * half;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (GR) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : s[kb][r] * c2;
      } else if (kb * 32 + 32 <= valid) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] *= c2;
      } else if (kb * 32 >= valid) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = -INFINITY;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) ? -INFINITY : s[kb][r] * c2;
      }
    }
  }

  // The running max m only has to keep the probabilities finite (p <= 2^64 here):
  // floating point does not care how far below 1 they are. O and l always share m,
  // so OUT = O / l and LSE = m + log2 l are exact whichever m is used.
  template <bool MASK, bool FIRST>
  __device__ __forceinline__ void softmax(int valid, float c2, int half) {
    if (MASK) {  // keys past the end of the partition
      // The mask is applied to scaled scores and the rest of the tile then runs with
      // a unit scale: masking raw scores to -inf would give -inf * 0 = NaN for a zero
      // softmax scale (or a zero fp8 factor), where every valid key must weigh e^0.
      // key = kb * 32 + 8 (r / 4) + 4 half + r % 4 >= valid, with the lane part moved to
      // the right: every comparison is an immediate against one register (per-key
      // indices would be hoisted out of the tile loop and held in ~30 VGPRs)
      mask_tail(valid, c2, half);
      c2 = 1.0f;
    }
    // Exponentiate first: the probabilities of the tile are taken with the running max
    // as it stands; only when some lane's sum of them exceeds 2^64 or is not finite (a
    // score more than 64 above m) is the tile taken again after moving m to the exact row
    // max. The row's first tile (m = -inf) moves m first. The common tile then needs no
    // max over its scores, and one vote of the wave.
    float t;
    if constexpr (FIRST) {
      move_max(c2);
      t = exp_pass(c2);
    } else {
      t = exp_pass(c2);
      if (__builtin_amdgcn_ballot_w64(!(t <= kRescaleLimit)) != 0) {
        move_max(c2);
        t = exp_pass(c2);
      }
    }
    l += t;
    if (GR) lp += t;
  }

  // m <- max(m, the exact row max of the tile's scaled scores); O, l (and lp) rescaled.
  __device__ __forceinline__ void move_max(float c2) {
    float x = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = fmaxf(x, s[0][r]);
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, s[kb][r]);
    const float mx = wave_max_halves(x) * c2;
    const float mn = fmaxf(m, mx);
    const float f = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first tile (m = -inf)
    m = mn;
    l *= f;
    if (GR) lp *= f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= f;
  }

  // P = exp2(c2 s - m) of the tile into pf (bf16); returns this lane's sum of the fp32
  // probabilities (summing their bf16 roundings would put the bf16 unit roundoff, 2^-8,
  // straight into LSE).
  __device__ __forceinline__ float exp_pass(float c2) {
    const float nm = -m;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 p;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * c + e], c2, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * c + e + 1], c2, nm));
          acc0 += p0;
          acc1 += p1;
          p[e] = (__bf16)p0;
          p[e + 1] = (__bf16)p1;
        }
        pf[kb][c] = p;
        // grouped launches: keep the bf16 packing of P in this phase (left alone, the
        // compiler sinks it past the barrier into the next MFMA phase, next to its use)
        if (GR) asm volatile("" : "+v"(pf[kb][c]));
      }
    return acc0 + acc1;
  }
};

// Grouped launches: walks the key tiles of the group's partitions in order, one tile per
// advance(); past the last one, valid() <= 0. The host packs each group's non-empty
// partitions, and the kernel copies the group's (first key, keys, caller's index)
// triples to LDS before the first tile, so a partition change reads LDS (in order with
// the operand reads) instead of issuing scalar loads in the tile loop. The common path
// of advance() is one compare and two scalar adds. Every field is wave-uniform.
template <int KB>
struct TileCursor {
  const int* tab;      // LDS: 3 ints per partition of the group
  int p, cnt;          // current partition (group-relative), partitions in the group
  int first, left;     // the current tile's first key, keys from it to the partition's end
  __device__ __forceinline__ void set(int q) {   // partition q (cnt: past the end)
    p = q;
    first = q < cnt ? __builtin_amdgcn_readfirstlane(tab[3 * q]) : 0;
    left = q < cnt ? __builtin_amdgcn_readfirstlane(tab[3 * q + 1]) : 0;
  }
  __device__ __forceinline__ void init(const int* table, int count) {
    tab = table;
    cnt = count;
    set(0);
  }
  __device__ __forceinline__ int first_key() const { return first; }
  __device__ __forceinline__ int valid() const { return left; }
  __device__ __forceinline__ bool last_of_partition() const { return left <= KB; }
  __device__ __forceinline__ int index() const { return __builtin_amdgcn_readfirstlane(tab[3 * p + 2]); }
  __device__ __forceinline__ void advance() {
    if (left > KB) {
      left -= KB;
      first += KB;
    } else if (p < cnt) {
      set(p + 1);
    }
  }
};

// Tile staging. Group 1 (waves 4-7) owns K: 16-byte chunks, D / 8 (bf16) or D / 16
// (fp8) lanes per row. Group 0 (waves 0-3) owns V: a unit is 4 keys x 8 d,
// transposed in registers and written as 8-byte key groups of 8 V^T rows; KB / 4
// consecutive lanes cover the key groups of one row. fp8 V (V8): a unit's 4 keys
// arrive as 8-byte loads of 8 E4M3 codes and are widened to bf16 (exact: every E4M3
// value is a bf16 value) before the same transposition, so LDS and the PV MFMA see
// bf16 V^T and the per-(b, h) factor of V is applied to OUT in the epilogue.
template <int D, bool QK8, bool V8 = false>
struct Stager {
  static constexpr int KCH = QK8 ? D / 16 : D / 8;  // 16-byte chunks per K row
  static constexpr int VCH = D / 8;                 // 16-byte chunks per V row
  static constexpr int GT = kThreads / 2;           // threads per group
  static constexpr int KB = Tile<D>::KB;
  static constexpr int KLOADS = KB * KCH / GT;      // K chunks per thread
  static constexpr int KROWS = GT / KCH;            // K rows per load round
  static constexpr int VUNITS = (KB / 4) * VCH;     // V units per tile
  static constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw 32-bit buffer, no swizzle
  u32x4 r[4];
  u32x2 r8[4];           // fp8 V: the 8 codes of each of the unit's 4 keys
  const char* src;       // K or V rows of this (b, h): from the partition's first key, or
                         // (grouped launches) from key 0
  int stride_bytes;      // between rows
  int row_bytes;         // D elements
  int n;                 // keys in the partition
  int voff[4];           // byte offsets of this thread's loads within a tile
  int w_off;             // LDS write base of this thread
  bool on;
  TileCursor<KB> cur;    // grouped launches: the next tile to load

  // Buffer resource covering exactly `rows` rows from key `first` (rows <= 0: an empty
  // range): loads past a partition's end are range-checked by the hardware and return
  // zeros, without a branch or a clamp per lane.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(int first, int rows) const {
    const int bytes = rows > 0 ? (min(rows, KB) - 1) * stride_bytes + row_bytes : 0;
    const uint64_t base = reinterpret_cast<uint64_t>(src + (int64_t)(rows > 0 ? first : 0) * stride_bytes);
    return make_rsrc(base, bytes);
  }
  // Grouped launches: the same without branches (rows <= 0 gives a zero-length range, whose
  // base address is then never dereferenced).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at_nb(int first, int rows) const {
    const int bytes = max((min(rows, KB) - 1) * stride_bytes + row_bytes, 0);
    const uint64_t base = reinterpret_cast<uint64_t>(src + (int64_t)first * stride_bytes);
    return make_rsrc(base, bytes);
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(uint64_t base, int bytes) const {
    // all of it is wave-uniform; readfirstlane keeps the descriptor in SGPRs
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
  }
  // tile `tile` of the partition (src at its first key)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(int tile) const {
    return rsrc_at(tile * KB, n - tile * KB);
  }
  // the cursor's tile, then one tile on (grouped launches)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t next_rsrc() {
    const __amdgpu_buffer_rsrc_t rs = rsrc_at_nb(cur.first_key(), cur.valid());
    cur.advance();
    return rs;
  }
  __device__ __forceinline__ void load_k_from(__amdgpu_buffer_rsrc_t rs) {
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[j], 0, 0);
  }
  __device__ __forceinline__ void load_k(int tile) { load_k_from(tile_rsrc(tile)); }
  __device__ __forceinline__ void load_v_from(__amdgpu_buffer_rsrc_t rs) {
    if (!on) return;
    if constexpr (V8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) r8[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff[j], 0, 0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[j], 0, 0);
    }
  }
  // 2 E4M3 codes (bytes 0-1, or 2-3 for HI, of x) as a bf16 pair, exactly
  template <bool HI>
  __device__ __forceinline__ static unsigned widen2(unsigned x) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
  }
  template <int SLOT>
  __device__ __forceinline__ void store_k(char* smem) {
    using L = Lds<D, QK8>;
#pragma unroll
    for (int j = 0; j < KLOADS; ++j)
      *reinterpret_cast<u32x4*>(smem + w_off + SLOT * L::KTILE + j * KROWS * L::KP) = r[j];
  }
  __device__ __forceinline__ void load_v(int tile) {
    if (!on) return;
    load_v_from(tile_rsrc(tile));
  }
  template <int SLOT>
  __device__ __forceinline__ void store_v(char* smem) {
    using L = Lds<D, QK8>;
    if (!on) return;
    if constexpr (V8) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r[j] = u32x4{widen2<false>(r8[j][0]), widen2<true>(r8[j][0]), widen2<false>(r8[j][1]), widen2<true>(r8[j][1])};
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const unsigned v0 = r[0][w], v1 = r[1][w], v2 = r[2][w], v3 = r[3][w];
      // d = 8c + 2w takes the low halves, d = 8c + 2w + 1 the high halves
      const u32x2 lo = {__builtin_amdgcn_perm(v1, v0, 0x05040100u), __builtin_amdgcn_perm(v3, v2, 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(v1, v0, 0x07060302u), __builtin_amdgcn_perm(v3, v2, 0x07060302u)};
      *reinterpret_cast<u32x2*>(smem + w_off + SLOT * L::VTILE + (2 * w) * L::VP) = lo;
      *reinterpret_cast<u32x2*>(smem + w_off + SLOT * L::VTILE + (2 * w + 1) * L::VP) = hi;
    }
  }
};

// OUT of a wave's 32 rows, ESZ bytes per element (4: fp32, 2: bf16, 1: fp8 codes): a lane
// holds 4-element pieces of one row (piece(db, j): d = 32 db + 8 j + 4 half of row l32, as
// one 16-, 8- or 4-byte value); stored as they are, every store instruction would write
// small pieces of 32 rows. Once the schedule's last barrier is passed the tile slots are
// free: each wave passes its rows through its own LDS region, PB bytes of a row at a time,
// and reads them back by rows, so that every store writes whole PB-byte row segments
// (128 or 256 bytes), streamed past the caches (nontemporal: written once).
// rows: the wave's rows inside the output (the others are not stored); out_rows: the
// first one; row_bytes: the output's row pitch.
template <int D, bool QK8, int ESZ, typename F>
__device__ __forceinline__ void store_rows(char* smem, int wave, int lane, char* out_rows, int rows, F piece) {
  using L = Lds<D, QK8>;
  constexpr int RB = D * ESZ;                                 // bytes of a row
  constexpr int PB = kWaves * kRowsPerWave * (RB + 16) <= L::BYTES ? RB
                     : kWaves * kRowsPerWave * (RB / 2 + 16) <= L::BYTES ? RB / 2 : RB / 4;
  constexpr int RP = PB + 16;                                 // LDS row pitch
  constexpr int LPR = PB / 16;                                // lanes per row when reading back
  constexpr int RPI = 64 / LPR;                               // rows per read
  constexpr int NDB = D / 32;
  static_assert(kWaves * kRowsPerWave * RP <= L::BYTES && RPI >= 1 && kRowsPerWave % RPI == 0, "epilogue staging");
  const int l32 = lane & 31, half = lane >> 5;
  char* reg = smem + wave * kRowsPerWave * RP;
#pragma unroll
  for (int pass = 0; pass < RB / PB; ++pass) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (db * 32 + 8 * j) * ESZ - pass * PB;   // the piece pair's first byte in the pass
        if (off >= 0 && off < PB) {
          const auto v = piece(db, j);
          using P = std::remove_cv_t<decltype(v)>;
          *reinterpret_cast<P*>(reg + l32 * RP + off + 4 * ESZ * half) = v;
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int it = 0; it < kRowsPerWave / RPI; ++it) {
      const int row = it * RPI + lane / LPR, col = lane % LPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + row * RP + col * 16);
      if (row < rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out_rows + (int64_t)row * RB + pass * PB + col * 16));
    }
    // the next pass rewrites the region: its reads are complete first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

// Schedule ("ping-pong"): the 8 waves form two groups of 4, one wave of each group
// per SIMD. Every wave alternates an MFMA phase X_t (S_t = K_t Q^T and
// O += V_{t-1} P_{t-1}^T) with a VALU phase Y_t (softmax of S_t -> P_t, plus tile
// staging), separated by workgroup barriers. Group 1 runs one phase behind group 0,
// so on each SIMD one wave is in its MFMA phase while the other is in its VALU
// phase (a wave does not overlap its own VALU work with its own MFMAs). Group 1
// stages K (tile t+2 during Y_t), group 0 stages V (tile t during Y_t); two LDS
// slots per operand suffice for this offset: a slot is rewritten only after both
// groups' last read of its previous tile.
//
// GROUPED: a workgroup walks the partitions of one group (a run of consecutive entries
// of the range list) one after the other with the same schedule, keeping O, the running
// max and the composed row sum in registers across them: the online softmax over the
// concatenated keys of the group is the composition of their states (DiTango review
// page, axiom ledger, Eq. 1-2; "If this is right": composed states merged into coarser
// groups). Each partition's LSE comes from a row sum restarted at the partition; the
// group's composed state is written once, optionally composed with a given state (a
// cached one) in the epilogue.
//
// OUT: kOutF32, kOutBF16, or kOutFP8: a state payload (E4M3 codes of OUT / f with one
// factor f = max|OUT| / 448 per row; single-partition launches only). V8: fp8 V (with
// QK8).
template <int D, int OUT, bool QK8, bool GROUPED = false, bool V8 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnArgs a) {
  using L = Lds<D, QK8>;
  using W = Wave<D, QK8, GROUPED>;
  using St = Stager<D, QK8, V8>;
  static_assert(kQB == 1 && St::KLOADS >= 1 && St::KLOADS <= 4 && St::VUNITS <= St::GT, "tile shape");
  static_assert(!(GROUPED && OUT != kOutF32), "grouped launches write fp32 states");
  static_assert(!V8 || QK8, "fp8 V comes with fp8 Q and K");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  // grouped launches: (first key, keys, caller's index) of every partition of the group
  __shared__ int gtab[GROUPED ? 3 * AS_MAX_PARTITIONS : 1];

  // Units (partition or group, b, h) are dealt round-robin over the 8 XCDs (workgroup i
  // runs on XCD i % 8) and the query tiles of a unit run consecutively on its XCD, whose L2
  // then serves their common K/V; listing long groups first runs them first everywhere.
  // A partial last query tile (Sq not a multiple of 256) has waves without rows, which
  // only stage, and takes less time than a full one. An XCD runs the full tiles of all
  // its units first and the partial ones after them (longest first), or, where the launch
  // found it cheaper (split_kr > 0), in the order under which the hardware's in-order
  // dispatch to free compute units keeps split_kr of them on partial tiles and the others
  // on full ones: full tile f starts at 16 * floor(f / (C - split_kr)) and partial tile r
  // at R16 * floor(r / split_kr) in units of a sixteenth of a full tile (R16 = 8 + the
  // partial tile's waves with rows), and workgroups are issued in that order (full first
  // on ties). The grid is padded to a multiple of 8 units.
  int qtile, bh, part;   // part: the partition, or for GROUPED the group
  {
    const int units = (GROUPED ? a.G : a.P) * a.B * a.H;
    const int x = blockIdx.x % 8, s = blockIdx.x / 8, ux = (units + 7) / 8;
    const int nf = a.Sq % kBQ ? a.n_qtiles - 1 : a.n_qtiles;   // full query tiles per unit
    int k;
    if (!GROUPED && a.split_kr > 0) {
      const int kr = a.split_kr, kf = a.split_c - kr;
      const int NF = ux * nf, NR = ux * (a.n_qtiles - nf);
      const int R16 = 8 + (a.Sq - nf * kBQ + kRowsPerWave - 1) / kRowsPerWave;
      // position of full tile f in the issue order: f plus the partial tiles that start
      // before it
      auto pos_f = [&](int f) {
        const int t = 16 * (f / kf);
        return f + min(NR, kr * ((t + R16 - 1) / R16));
      };
      int lo = 0, hi = NF;   // g = number of full tiles at positions <= s
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pos_f(mid) <= s) lo = mid + 1;
        else hi = mid;
      }
      if (lo > 0 && pos_f(lo - 1) == s) {
        k = (lo - 1) / nf;
        qtile = lo - 1 - k * nf;
      } else {
        k = s - lo;
        qtile = a.n_qtiles - 1;
      }
    } else if (s < ux * nf) {
      k = s / nf;
      qtile = s - k * nf;
    } else {
      k = s - ux * nf;
      qtile = a.n_qtiles - 1;
    }
    const int j = x + 8 * k;
    if (j >= units) return;
    bh = j % (a.B * a.H);
    part = j / (a.B * a.H);
  }
  const int b = bh / a.H, hh = bh % a.H;
  if constexpr (!GROUPED) {
    AS_STAMP(0, __builtin_amdgcn_s_memrealtime());
    AS_STAMP(4, __builtin_amdgcn_s_memtime());
    AS_STAMP(6, (unsigned long long)qtile | ((unsigned long long)part << 32));
    AS_STAMP(7, __builtin_amdgcn_s_getreg((31 << 11) | 4) | ((unsigned long long)__builtin_amdgcn_s_getreg((31 << 11) | 20) << 32));
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, half = lane >> 5;
  // wave-uniform; readfirstlane lets the compiler keep group-dependent values in SGPRs
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int gtid = tid & (St::GT - 1);

  const int q0 = qtile * kBQ;
  const int64_t row_base = ((int64_t)part * a.B * a.H + bh) * a.Sq;   // row index in out/lse
  float* __restrict__ lse = a.lse + row_base;
  int n = 0;
  if constexpr (!GROUPED) {
    n = a.ranges[2 * part + 1] - a.ranges[2 * part];
    if (n <= 0) {  // empty partition: the identity state (0, -inf)
      for (int r = tid; r < kBQ; r += kThreads) {
        const int q = q0 + r;
        if (q < a.Sq) {
          lse[q] = -INFINITY;
          if constexpr (OUT == kOutFP8) {   // codes 0, factor 0
            char* pay = static_cast<char*>(a.out) + (int64_t)part * a.payload_bytes;
            const int64_t srow = (int64_t)bh * a.Sq + q;
            for (int c = 0; c < D / 16; ++c) *reinterpret_cast<u32x4*>(pay + srow * D + 16 * c) = u32x4{0u, 0u, 0u, 0u};
            reinterpret_cast<float*>(pay + a.state_rows * D)[srow] = 0.f;
          } else {
            for (int c = 0; c < D / 4; ++c) store_out4<OUT>(a.out, (row_base + q) * D + 4 * c, f32x4{0.f, 0.f, 0.f, 0.f});
          }
        }
      }
      return;
    }
  }

  W w;
  const int qrow = q0 + wave * kRowsPerWave + l32;
  // fp8 scores are in units of the two dequantisation factors of this (b, h)
  float c2 = QK8 ? a.scale_log2 * a.q_scale[bh] * a.k_scale[bh] : a.scale_log2;
  if constexpr (QK8) {
    // A negative product of the factors is moved into Q: flipping the sign bit of every
    // E4M3 code negates its value exactly, and the softmax then sees a scale >= 0 (its
    // per-tile maximum of raw scores is the maximum of the scaled ones).
    const unsigned qsign = c2 < 0.f ? 0x80808080u : 0u;
    c2 = fabsf(c2);
    const unsigned char* qp = reinterpret_cast<const unsigned char*>(a.q) + b * a.q_sb + hh * a.q_sh +
                              (int64_t)min(qrow, a.Sq - 1) * a.q_ss + 32 * half;
#pragma unroll
    for (int ds = 0; ds < W::NDS; ++ds) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qp + 64 * ds);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qp + 64 * ds + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w.qf.v[ds][e] = qrow < a.Sq ? (int)(x0[e] ^ qsign) : 0;
        w.qf.v[ds][4 + e] = qrow < a.Sq ? (int)(x1[e] ^ qsign) : 0;
      }
    }
  } else {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb + hh * a.q_sh;
#pragma unroll
    for (int ds = 0; ds < W::NDS; ++ds) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qp + (int64_t)min(qrow, a.Sq - 1) * a.q_ss + ds * 16 + 8 * half);
      w.qf.v[ds] = __builtin_bit_cast(bf16x8, qrow < a.Sq ? x : u32x4{0u, 0u, 0u, 0u});
    }
  }
#pragma unroll
  for (int db = 0; db < W::NDB; ++db) w.o[db] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < W::NKB; ++kb)
#pragma unroll
    for (int c = 0; c < 2; ++c) w.pf[kb][c] = bf16x8{};
  w.m = -INFINITY;
  w.l = 0.f;
  w.lp = 0.f;
  w.k_rd = l32 * L::KP + (QK8 ? 32 : 16) * half;
  w.v_rd = L::V0 + l32 * L::VP + 16 * half;
  constexpr int KB = Tile<D>::KB;

  St st;
  // this (b, h)'s K (group 1) or V (group 0) rows; a partition starts ks rows further
  const int64_t kv_bh = b * a.k_sb + hh * a.k_sh;   // elements
  const char* kv_base;
  if (grp == 1) {
    constexpr int ek = QK8 ? 1 : 2;   // bytes per K element
    st.stride_bytes = (int)(a.k_ss * ek);
    st.row_bytes = D * ek;
    kv_base = reinterpret_cast<const char*>(a.k) + kv_bh * ek;
    const int row = gtid / St::KCH, ch = gtid % St::KCH;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.voff[j] = (row + j * St::KROWS) * st.stride_bytes + ch * 16;
    st.w_off = row * L::KP + ch * 16;
    st.on = true;
  } else {
    constexpr int ev = V8 ? 1 : 2;    // bytes per V element
    st.stride_bytes = (int)(a.k_ss * ev);
    st.row_bytes = D * ev;
    kv_base = reinterpret_cast<const char*>(a.v) + kv_bh * ev;
    const int va = gtid % (KB / 4), vc = gtid / (KB / 4);   // 4-key group, 8-wide d chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) st.voff[j] = (4 * va + j) * st.stride_bytes + vc * 8 * ev;
    st.w_off = L::V0 + (8 * vc) * L::VP + vt_group_pos(va);
    st.on = gtid < St::VUNITS;
  }
  st.stride_bytes = __builtin_amdgcn_readfirstlane(st.stride_bytes);
  st.row_bytes = __builtin_amdgcn_readfirstlane(st.row_bytes);
  // Points the stager at the ks-th row of this (b, h); wave-uniform, so that the
  // per-tile descriptor arithmetic runs on the scalar unit.
  auto start_partition = [&](int ks_, int n_) __attribute__((always_inline)) {
    const uint64_t p = reinterpret_cast<uint64_t>(kv_base + (int64_t)ks_ * st.stride_bytes);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    st.src = reinterpret_cast<const char*>(lo | (hi << 32));
    st.n = __builtin_amdgcn_readfirstlane(n_);
  };
  int T = 0;   // key tiles of the partition, or of all partitions of the group

  // Grouped launches run one schedule over the tiles of all the group's partitions in a
  // row (one pipeline fill per group); the stagers and the softmax each follow them with
  // a cursor. After the softmax of a partition's last tile its row sum is complete: its
  // LSE is written and the partition sum restarts.
  TileCursor<KB> sc;   // softmax cursor (grouped launches)
  if constexpr (GROUPED) {
    // readfirstlane: the group's bounds and ranges are uniform; without it the code that
    // depends on them would be compiled as divergent
    const int p0 = __builtin_amdgcn_readfirstlane(a.group_starts[part]);
    const int p1 = __builtin_amdgcn_readfirstlane(a.group_starts[part + 1]);
    for (int p = p0; p < p1; ++p) {   // packed ranges: every one non-empty
      const int n_ = __builtin_amdgcn_readfirstlane(a.ranges[2 * p + 1]) - __builtin_amdgcn_readfirstlane(a.ranges[2 * p]);
      T += (n_ + KB - 1) / KB;
    }
    for (int i = tid; i < p1 - p0; i += kThreads) {
      gtab[3 * i] = a.ranges[2 * (p0 + i)];
      gtab[3 * i + 1] = a.ranges[2 * (p0 + i) + 1] - a.ranges[2 * (p0 + i)];
      gtab[3 * i + 2] = a.part_index[p0 + i];
    }
    __syncthreads();
    start_partition(0, 0);   // src = key 0 of this (b, h); tiles come from the cursor
    st.cur.init(gtab, p1 - p0);
    sc.init(gtab, p1 - p0);
  }
  auto LDK = [&](int tile) __attribute__((always_inline)) {
    if constexpr (GROUPED) st.load_k_from(st.next_rsrc());
    else st.load_k(tile);
  };
  auto LDV = [&](int tile) __attribute__((always_inline)) {
    if constexpr (GROUPED) st.load_v_from(st.next_rsrc());
    else st.load_v(tile);
  };
  auto SMX = [&](int tile, auto FIRSTC) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(FIRSTC)::value;
    if constexpr (GROUPED) {
      w.template softmax_phase<FIRST>(sc.valid(), c2, half);
      if (sc.last_of_partition()) {
        // The partition's sum is taken against the group's running max: a partition whose
        // every score lies more than 126 below it (log2 units) sums to 0 here, and its LSE
        // comes out as -inf (its weight against the group's is under 2^-126 either way).
        const float lp = wave_sum_halves(w.lp);
        if (a.part_lse && qrow < a.Sq && half == 0) {
          const int orig = sc.index();   // the caller's partition index
          a.part_lse[((int64_t)orig * a.B * a.H + bh) * a.Sq + qrow] = (w.m + __log2f(lp)) * 0.69314718055994530942f;
        }
        w.lp = 0.f;
      }
      sc.advance();
    } else {
      w.template softmax_phase<FIRST>(n - tile * KB, c2, half);
    }
  };

  // The schedule of one partition (n keys, T tiles); ON = false is the copy for a wave
  // whose 32 rows all lie past Sq (last query tile): it only stages and passes the same
  // barriers.
  auto schedule = [&](auto ONC) __attribute__((always_inline)) {
    constexpr bool ON = decltype(ONC)::value;
    // Both groups pass 2T + 3 barriers: group 1's extra leading phase (staging
    // K tile 1) is matched by group 0's trailing empty phase.
    if (grp == 1) {
      LDK(0);
      st.template store_k<0>(smem);
      LDK(1);
      lds_barrier();                                   // K tile 0 visible
      if (T > 1) st.template store_k<1>(smem);         // phase Y_{-1}
      LDK(2);
      lds_barrier();
      if constexpr (ON) w.template mfma_phase<0, 0, true, false>(smem);  // X_0
      lds_barrier();
      if constexpr (ON) SMX(0, std::true_type{});                    // Y_0
      if (T > 2) st.template store_k<0>(smem);
      LDK(3);
      lds_barrier();
      int t = 1;
      for (; t + 1 < T; t += 2) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);     // X_t, t odd
        lds_barrier();
        if constexpr (ON) SMX(t, std::false_type{});
        if (t + 2 < T) st.template store_k<1>(smem);
        LDK(t + 3);
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, true, true>(smem);     // X_{t+1}, even
        lds_barrier();
        if constexpr (ON) SMX(t + 1, std::false_type{});
        if (t + 3 < T) st.template store_k<0>(smem);
        LDK(t + 4);
        lds_barrier();
      }
      if (t < T) {  // t odd, last tile
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) SMX(t, std::false_type{});
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, false, true>(smem);    // X_T, V slot (T-1)&1 = 1
      } else {      // T even (or 1): V slot (T-1)&1
        if constexpr (ON) {
          if (T & 1) w.template mfma_phase<0, 0, false, true>(smem);
          else w.template mfma_phase<0, 1, false, true>(smem);
        }
      }
      lds_barrier();
    } else {
      LDV(0);
      lds_barrier();
      if constexpr (!GROUPED) AS_STAMP(1, __builtin_amdgcn_s_memrealtime());
      if constexpr (ON) w.template mfma_phase<0, 0, true, false>(smem);  // X_0
      lds_barrier();
      if constexpr (ON) SMX(0, std::true_type{});                    // Y_0
      st.template store_v<0>(smem);
      LDV(1);
      lds_barrier();
      int t = 1;
      for (; t + 1 < T; t += 2) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) SMX(t, std::false_type{});
        st.template store_v<1>(smem);
        LDV(t + 1);
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, true, true>(smem);
        lds_barrier();
        if constexpr (ON) SMX(t + 1, std::false_type{});
        st.template store_v<0>(smem);
        LDV(t + 2);
        lds_barrier();
      }
      if (t < T) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) SMX(t, std::false_type{});
        st.template store_v<1>(smem);
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, false, true>(smem);
      } else {
        if constexpr (ON) {
          if (T & 1) w.template mfma_phase<0, 0, false, true>(smem);
          else w.template mfma_phase<0, 1, false, true>(smem);
        }
      }
      lds_barrier();
      lds_barrier();   // group 1's trailing X_T phase
    }
  };

  if constexpr (GROUPED) {
    if (T > 0) {
      if (__builtin_amdgcn_readfirstlane(q0 + wave * kRowsPerWave) < a.Sq) schedule(std::true_type{});
      else schedule(std::false_type{});
    }

    // ---- epilogue: the group's composed state, composed with the given state for group 0
    const float lt = wave_sum_halves(w.l);
    // weight of O (fp8 V: O is in units of V's factor)
    float wo = lt > 0.f ? (V8 ? a.v_scale[bh] : 1.0f) / lt : 0.f;
    float L = lt > 0.f ? (w.m + __log2f(lt)) * 0.69314718055994530942f : -INFINITY;
    float wc = 0.f;                            // weight of the given state's OUT
    const bool fold = a.fold_out != nullptr && part == 0 && qrow < a.Sq;
    const int64_t frow = (int64_t)bh * a.Sq + qrow;   // row of the given [B][H][Sq] state
    if (fold) {
      const float Lc = a.fold_lse[frow];
      const float M = fmaxf(L, Lc);
      if (M == -INFINITY) {
        wo = 0.f;
        L = -INFINITY;
      } else {
        const float e1 = expf(L - M), e2 = expf(Lc - M), S = e1 + e2;
        wo *= e1 / S;
        wc = e2 / S;
        L = M + logf(S);
      }
    }
    const int w0 = q0 + wave * kRowsPerWave;     // the wave's first row
    store_rows<D, QK8, 4>(smem, wave, lane, reinterpret_cast<char*>(static_cast<float*>(a.out) + (row_base + w0) * D), a.Sq - w0,
                           [&](int db, int j) __attribute__((always_inline)) {
                             f32x4 val = {w.o[db][4 * j] * wo, w.o[db][4 * j + 1] * wo, w.o[db][4 * j + 2] * wo,
                                          w.o[db][4 * j + 3] * wo};
                             if (fold) {
                               const f32x4 c = *reinterpret_cast<const f32x4*>(a.fold_out + frow * D + db * 32 +
                                                                               8 * j + 4 * half);
                               val = f32x4{__builtin_fmaf(wc, c[0], val[0]), __builtin_fmaf(wc, c[1], val[1]),
                                           __builtin_fmaf(wc, c[2], val[2]), __builtin_fmaf(wc, c[3], val[3])};
                             }
                             return val;
                           });
    if (half == 0 && qrow < a.Sq) lse[qrow] = L;
  } else {
    const int ks = a.ranges[2 * part];
    T = (n + KB - 1) / KB;
    start_partition(ks, n);
    if (__builtin_amdgcn_readfirstlane(q0 + wave * kRowsPerWave) < a.Sq) schedule(std::true_type{});
    else schedule(std::false_type{});
    AS_STAMP(2, __builtin_amdgcn_s_memrealtime());

    // ---- epilogue: OUT = O / l, LSE = (m + log2 l) ln 2
    const float lt = wave_sum_halves(w.l);
    const float inv = (V8 ? a.v_scale[bh] : 1.0f) / lt;   // fp8 V: O is in units of V's factor
    if constexpr (OUT == kOutFP8) {
      // The row's largest |OUT| (the two halves of a row hold its two halves of D); OUT
      // is stored as the E4M3 codes of OUT * (448 / amax), rounded to nearest even, with
      // the factor amax / 448 (0 for a zero row, whose codes are 0).
      float mx = 0.f;
#pragma unroll
      for (int db = 0; db < W::NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(w.o[db][e]));
      const float amax = wave_max_halves(mx) * fabsf(inv);   // = max |O * inv|: rounding is monotone
      const float qf = amax > 0.f ? 448.0f / amax : 0.f;
      char* pay = static_cast<char*>(a.out) + (int64_t)part * a.payload_bytes;
      const int w0 = q0 + wave * kRowsPerWave;   // the wave's first row
      store_rows<D, QK8, 1>(smem, wave, lane, pay + ((int64_t)bh * a.Sq + w0) * D, a.Sq - w0,
                            [&](int db, int j) __attribute__((always_inline)) {
                              float x[4];
#pragma unroll
                              for (int e = 0; e < 4; ++e) x[e] = clamp448((w.o[db][4 * j + e] * inv) * qf);
                              return fp8x4(x[0], x[1], x[2], x[3]);
                            });
      if (half == 0 && qrow < a.Sq) {
        reinterpret_cast<float*>(pay + a.state_rows * D)[(int64_t)bh * a.Sq + qrow] = amax / 448.0f;
        lse[qrow] = (w.m + __log2f(lt)) * 0.69314718055994530942f;
      }
    } else {
      // fp32 or bf16 (rounded to nearest even) OUT
      constexpr int ESZ = OUT == kOutBF16 ? 2 : 4;
      const int w0 = q0 + wave * kRowsPerWave;   // the wave's first row
      store_rows<D, QK8, ESZ>(smem, wave, lane, static_cast<char*>(a.out) + (row_base + w0) * D * ESZ, a.Sq - w0,
                              [&](int db, int j) __attribute__((always_inline)) {
                                const f32x4 v = {w.o[db][4 * j] * inv, w.o[db][4 * j + 1] * inv,
                                                 w.o[db][4 * j + 2] * inv, w.o[db][4 * j + 3] * inv};
                                if constexpr (OUT == kOutBF16) {
                                  const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                                  return __builtin_bit_cast(u32x2, h);
                                } else {
                                  return v;
                                }
                              });
      if (half == 0 && qrow < a.Sq) lse[qrow] = (w.m + __log2f(lt)) * 0.69314718055994530942f;
    }
  }
#ifdef AS_WG_STAMPS
  if constexpr (!GROUPED) {
    __syncthreads();
    AS_STAMP(3, __builtin_amdgcn_s_memrealtime());
    AS_STAMP(5, __builtin_amdgcn_s_memtime());
  }
#endif
}

// Launch of one instance: D from the arguments, OUT from a.out_kind (single-partition
// launches; grouped ones write fp32 states).
template <int D, int OUT, bool QK8, bool GROUPED, bool V8>
hipError_t launch_instance(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, OUT, QK8, GROUPED, V8>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Issue order of a single-partition launch with partial query tiles (one workgroup per
// compute unit: the kernel's registers allow no second). Costs in sixteenths of a full
// tile: a full tile 16, a partial one R16. Longest first (full tiles, then partial ones)
// leaves, per XCD of C compute units, about the load of the greedy assignment computed
// below as `lpt`; keeping kr units on partial tiles and the others on full ones costs
// max(16 ceil(NF / (C - kr)), R16 ceil(NR / kr)). The split with the least cost is taken
// where it beats longest first (split_kr = kr), else split_kr = 0.
inline void plan_issue_order(AttnArgs& a) {
  a.split_kr = 0;
  a.split_c = device_cus() / 8;
  const int C = a.split_c;
  const int nf = a.Sq % kBQ ? a.n_qtiles - 1 : a.n_qtiles;
  const int64_t ux = ((int64_t)a.P * a.B * a.H + 7) / 8;
  const int64_t NF = ux * nf, NR = ux * (a.n_qtiles - nf);
  // long lists (many rounds) lose little to the last round: no planning
  if (NR == 0 || NF == 0 || C < 2 || NF + NR > 4096) return;
  const int64_t R16 = 8 + (a.Sq - nf * kBQ + kRowsPerWave - 1) / kRowsPerWave;
  // the last plan, for repeated launches of one shape
  thread_local int64_t key[4] = {-1, -1, -1, -1};
  thread_local int kr_last = 0;
  if (key[0] == NF && key[1] == NR && key[2] == R16 && key[3] == C) {
    a.split_kr = kr_last;
    return;
  }
  // greedy longest first: each tile to the least loaded unit (a min-heap of loads)
  std::vector<int64_t> load(C, 0);
  for (int64_t i = 0; i < NF + NR; ++i) {
    std::pop_heap(load.begin(), load.end(), std::greater<int64_t>());
    load.back() += i < NF ? 16 : R16;
    std::push_heap(load.begin(), load.end(), std::greater<int64_t>());
  }
  int64_t best = *std::max_element(load.begin(), load.end());
  for (int k = 1; k < C; ++k) {
    const int64_t cost = std::max(16 * ((NF + C - k - 1) / (C - k)), R16 * ((NR + k - 1) / k));
    if (cost < best) {
      best = cost;
      a.split_kr = k;
    }
  }
  key[0] = NF;
  key[1] = NR;
  key[2] = R16;
  key[3] = C;
  kr_last = a.split_kr;
}

template <int D, bool QK8, bool GROUPED, bool V8>
hipError_t launch_for_d(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if constexpr (GROUPED) {
    return launch_instance<D, kOutF32, QK8, true, V8>(a, grid, stream);
  } else {
    AttnArgs b = a;
    plan_issue_order(b);
    switch (b.out_kind) {
      case kOutF32: return launch_instance<D, kOutF32, QK8, false, V8>(b, grid, stream);
      case kOutBF16: return launch_instance<D, kOutBF16, QK8, false, V8>(b, grid, stream);
      case kOutFP8: return launch_instance<D, kOutFP8, QK8, false, V8>(b, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template <bool QK8, bool GROUPED, bool V8>
hipError_t launch_variant(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if (a.D == 128) return launch_for_d<128, QK8, GROUPED, V8>(a, grid, stream);
  if (a.D == 64) return launch_for_d<64, QK8, GROUPED, V8>(a, grid, stream);
  return hipErrorInvalidValue;
}

// Grid of a launch: units (partition, b, h), or (group, b, h) for a grouped one, padded to
// a multiple of 8 (the kernel's XCD mapping), times query tiles. Zero blocks: nothing to
// launch; -1: too many.
inline int64_t attn_grid(const AttnArgs& a, bool grouped) {
  const int64_t total = ((int64_t)(grouped ? a.G : a.P) * a.B * a.H + 7) / 8 * 8 * a.n_qtiles;
  return total > 0x7fffffff ? -1 : total;
}

}  // namespace
}  // namespace as
