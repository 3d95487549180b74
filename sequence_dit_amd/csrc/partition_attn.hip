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
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

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

// Stores of OUT elements: fp32, or bf16 rounded to nearest even.
template <bool BF16>
__device__ __forceinline__ void store_out4(void* base, int64_t off, f32x4 v) {
  if (BF16) {
    const bf16x4 h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(base) + off) = __builtin_bit_cast(u32x2, h);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = v;
  }
}

template <bool BF16>
__device__ __forceinline__ void store_out1(void* base, int64_t off, float v) {
  if (BF16) static_cast<__bf16*>(base)[off] = (__bf16)v;
  else static_cast<float*>(base)[off] = v;
}

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
constexpr float kRescaleThreshold = 64.0f;   // log2 units: probabilities stay <= 2^64

// Maps the hardware workgroup id to a logical tile id so that consecutive logical
// ids land on the same XCD (workgroups are dealt round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int x = L % kXcd, idx = L / kXcd;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

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

// Per-wave state of the bf16 kernel; one wave owns 32 query rows.
template <int D, bool QK8>
struct Wave {
  static constexpr int NDS = QK8 ? D / 64 : D / 16;   // MFMA k-steps of S^T = K Q^T
  static constexpr int NDB = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int KB = Tile<D>::KB, NKB = Tile<D>::NKB;
  QFrag<D, QK8> qf;      // Q, for the whole partition
  f32x16 s[NKB];         // S^T of the current tile: [kb], reg r <-> key 32kb + 8(r/4) + 4half + r%4
  bf16x8 pf[NKB][2];     // P of the previous tile, B operand of O^T: [kb][c]
  f32x16 o[NDB];         // O^T: [db], reg r <-> d = 32db + 8(r/4) + 4half + r%4
  float m, l;            // running max (log2 domain, scaled) and row sum
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
  __device__ __forceinline__ void softmax_phase(int valid, float c2, int half) {
    if (valid < KB) softmax<true>(valid, c2, half);
    else softmax<false>(valid, c2, half);
  }

  // The running max m only has to keep the probabilities finite (p <= 2^64 here):
  // floating point does not care how far below 1 they are. Each lane compares its
  // own scores against m + 64 (one max3 chain, no cross-lane step); only when some
  // lane exceeds it (always on the first tile, where m = -inf) does the wave take
  // the exact row max, rescale O and l, and move m. O and l always share m, so
  // OUT = O / l and LSE = m + log2 l are exact whichever m is used.
  template <bool MASK>
  __device__ __forceinline__ void softmax(int valid, float c2, int half) {
    if (MASK) {  // keys past the end of the partition
      // key = kb * 32 + 8 (r / 4) + 4 half + r % 4 >= valid, with the lane part moved to
      // the right: every comparison is an immediate against one register (per-key
      // indices would be hoisted out of the tile loop and held in ~30 VGPRs)
      const int lim = valid - 4 * half;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) s[kb][r] = -INFINITY;
    }
    float x = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) x = fmaxf(x, s[0][r]);
#pragma unroll
    for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, s[kb][r]);
    if (__builtin_amdgcn_ballot_w64(x * c2 > m + kRescaleThreshold) != 0) {
      const float mx = wave_max_halves(x) * c2;
      const float mn = fmaxf(m, mx);
      const float f = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first tile (m = -inf)
      m = mn;
      l *= f;
      // in-place multiplies keep the accumulators in their registers across the branch
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(o[db][r]) : "v"(f));
    }
    const float nm = -m;
    // the row sum uses the fp32 probabilities: summing their bf16 roundings
    // would put the bf16 unit roundoff (2^-8) straight into LSE
    float acc0 = l, acc1 = 0.f;
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
      }
    l = acc0 + acc1;
  }
};

// Tile staging. Group 1 (waves 4-7) owns K: 16-byte chunks, D / 8 (bf16) or D / 16
// (fp8) lanes per row. Group 0 (waves 0-3) owns V: a unit is 4 keys x 8 d,
// transposed in registers and written as 8-byte key groups of 8 V^T rows; KB / 4
// consecutive lanes cover the key groups of one row.
template <int D, bool QK8>
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
  const char* src;       // K or V rows of this (b, h) starting at the partition
  int stride_bytes;      // between rows
  int row_bytes;         // D elements
  int n;                 // keys in the partition
  int voff[4];           // byte offsets of this thread's loads within a tile
  int w_off;             // LDS write base of this thread
  bool on;

  // Buffer resource covering exactly the valid rows of tile `tile`: loads past the
  // partition's end are range-checked by the hardware and return zeros, without a
  // branch or a clamp per lane. A tile past the end gets an empty range.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(int tile) const {
    const int rows = n - tile * KB;
    const int bytes = rows > 0 ? (min(rows, KB) - 1) * stride_bytes + row_bytes : 0;
    const uint64_t base = reinterpret_cast<uint64_t>(src + (int64_t)(rows > 0 ? tile * KB : 0) * stride_bytes);
    // all of it is wave-uniform; readfirstlane keeps the descriptor in SGPRs
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
  }
  __device__ __forceinline__ void load_k(int tile) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile);
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[j], 0, 0);
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
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[j], 0, 0);
  }
  template <int SLOT>
  __device__ __forceinline__ void store_v(char* smem) {
    using L = Lds<D, QK8>;
    if (!on) return;
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

// Schedule ("ping-pong"): the 8 waves form two groups of 4, one wave of each group
// per SIMD. Every wave alternates an MFMA phase X_t (S_t = K_t Q^T and
// O += V_{t-1} P_{t-1}^T) with a VALU phase Y_t (softmax of S_t -> P_t, plus tile
// staging), separated by workgroup barriers. Group 1 runs one phase behind group 0,
// so on each SIMD one wave is in its MFMA phase while the other is in its VALU
// phase (a wave does not overlap its own VALU work with its own MFMAs). Group 1
// stages K (tile t+2 during Y_t), group 0 stages V (tile t during Y_t); two LDS
// slots per operand suffice for this offset: a slot is rewritten only after both
// groups' last read of its previous tile.
template <int D, bool OUT_BF16, bool QK8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnArgs a) {
  using L = Lds<D, QK8>;
  using W = Wave<D, QK8>;
  using St = Stager<D, QK8>;
  static_assert(kQB == 1 && St::KLOADS >= 1 && St::KLOADS <= 4 && St::VUNITS <= St::GT, "tile shape");
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

  const int total = a.n_qtiles * a.B * a.H * a.P;
  const int lid = xcd_remap(blockIdx.x, total);
  const int qtile = lid % a.n_qtiles;
  const int rest = lid / a.n_qtiles;
  const int bh = rest % (a.B * a.H);
  const int part = rest / (a.B * a.H);
  const int b = bh / a.H, hh = bh % a.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, half = lane >> 5;
  // wave-uniform; readfirstlane lets the compiler keep group-dependent values in SGPRs
  const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int gtid = tid & (St::GT - 1);

  const int ks = a.ranges[2 * part], ke = a.ranges[2 * part + 1];
  const int n = ke - ks;
  const int q0 = qtile * kBQ;
  const int64_t row_base = ((int64_t)part * a.B * a.H + bh) * a.Sq;   // row index in out/lse
  float* __restrict__ lse = a.lse + row_base;

  if (n <= 0) {  // empty partition: the identity state (0, -inf)
    for (int r = tid; r < kBQ; r += kThreads) {
      const int q = q0 + r;
      if (q < a.Sq) {
        lse[q] = -INFINITY;
        for (int c = 0; c < D / 4; ++c) store_out4<OUT_BF16>(a.out, (row_base + q) * D + 4 * c, f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
    return;
  }

  W w;
  const int qrow = q0 + wave * kRowsPerWave + l32;
  if constexpr (QK8) {
    const unsigned char* qp = reinterpret_cast<const unsigned char*>(a.q) + b * a.q_sb + hh * a.q_sh +
                              (int64_t)min(qrow, a.Sq - 1) * a.q_ss + 32 * half;
#pragma unroll
    for (int ds = 0; ds < W::NDS; ++ds) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qp + 64 * ds);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qp + 64 * ds + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w.qf.v[ds][e] = qrow < a.Sq ? (int)x0[e] : 0;
        w.qf.v[ds][4 + e] = qrow < a.Sq ? (int)x1[e] : 0;
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
  w.k_rd = l32 * L::KP + (QK8 ? 32 : 16) * half;
  w.v_rd = L::V0 + l32 * L::VP + 16 * half;
  // fp8 scores are in units of the two dequantisation factors of this (b, h)
  const float c2 = QK8 ? a.scale_log2 * a.q_scale[bh] * a.k_scale[bh] : a.scale_log2;
  constexpr int KB = Tile<D>::KB;
  const int T = (n + KB - 1) / KB;

  St st;
  st.n = n;
  const int64_t kv_off = b * a.k_sb + hh * a.k_sh + (int64_t)ks * a.k_ss;   // elements
  if (grp == 1) {
    constexpr int ek = QK8 ? 1 : 2;   // bytes per K element
    st.stride_bytes = (int)(a.k_ss * ek);
    st.row_bytes = D * ek;
    st.src = reinterpret_cast<const char*>(a.k) + kv_off * ek;
    const int row = gtid / St::KCH, ch = gtid % St::KCH;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.voff[j] = (row + j * St::KROWS) * st.stride_bytes + ch * 16;
    st.w_off = row * L::KP + ch * 16;
    st.on = true;
  } else {
    st.stride_bytes = (int)(a.k_ss * 2);
    st.row_bytes = D * 2;
    st.src = reinterpret_cast<const char*>(a.v) + kv_off * 2;
    const int va = gtid % (KB / 4), vc = gtid / (KB / 4);   // 4-key group, 8-wide d chunk
#pragma unroll
    for (int j = 0; j < 4; ++j) st.voff[j] = (4 * va + j) * st.stride_bytes + vc * 16;
    st.w_off = L::V0 + (8 * vc) * L::VP + vt_group_pos(va);
    st.on = gtid < St::VUNITS;
  }
  // wave-uniform: the per-tile descriptor arithmetic then runs on the scalar unit
  {
    const uint64_t p = reinterpret_cast<uint64_t>(st.src);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    st.src = reinterpret_cast<const char*>(lo | (hi << 32));
    st.stride_bytes = __builtin_amdgcn_readfirstlane(st.stride_bytes);
    st.row_bytes = __builtin_amdgcn_readfirstlane(st.row_bytes);
    st.n = __builtin_amdgcn_readfirstlane(st.n);
  }

  // The schedule; ON = false is the copy for a wave whose 32 rows all lie past Sq
  // (last query tile): it only stages and passes the same barriers.
  auto schedule = [&](auto ONC) {
    constexpr bool ON = decltype(ONC)::value;
    // Both groups pass 2T + 3 barriers: group 1's extra leading phase (staging
    // K tile 1) is matched by group 0's trailing empty phase.
    if (grp == 1) {
      st.load_k(0);
      st.template store_k<0>(smem);
      st.load_k(1);
      lds_barrier();                                   // K tile 0 visible
      if (T > 1) st.template store_k<1>(smem);         // phase Y_{-1}
      st.load_k(2);
      lds_barrier();
      if constexpr (ON) w.template mfma_phase<0, 0, true, false>(smem);  // X_0
      lds_barrier();
      if constexpr (ON) w.softmax_phase(n, c2, half);                    // Y_0
      if (T > 2) st.template store_k<0>(smem);
      st.load_k(3);
      lds_barrier();
      int t = 1;
      for (; t + 1 < T; t += 2) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);     // X_t, t odd
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - t * KB, c2, half);
        if (t + 2 < T) st.template store_k<1>(smem);
        st.load_k(t + 3);
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, true, true>(smem);     // X_{t+1}, even
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - (t + 1) * KB, c2, half);
        if (t + 3 < T) st.template store_k<0>(smem);
        st.load_k(t + 4);
        lds_barrier();
      }
      if (t < T) {  // t odd, last tile
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - t * KB, c2, half);
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
      st.load_v(0);
      lds_barrier();
      if constexpr (ON) w.template mfma_phase<0, 0, true, false>(smem);  // X_0
      lds_barrier();
      if constexpr (ON) w.softmax_phase(n, c2, half);                    // Y_0
      st.template store_v<0>(smem);
      st.load_v(1);
      lds_barrier();
      int t = 1;
      for (; t + 1 < T; t += 2) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - t * KB, c2, half);
        st.template store_v<1>(smem);
        st.load_v(t + 1);
        lds_barrier();
        if constexpr (ON) w.template mfma_phase<0, 1, true, true>(smem);
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - (t + 1) * KB, c2, half);
        st.template store_v<0>(smem);
        st.load_v(t + 2);
        lds_barrier();
      }
      if (t < T) {
        if constexpr (ON) w.template mfma_phase<1, 0, true, true>(smem);
        lds_barrier();
        if constexpr (ON) w.softmax_phase(n - t * KB, c2, half);
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
  if (__builtin_amdgcn_readfirstlane(q0 + wave * kRowsPerWave) < a.Sq) schedule(std::true_type{});
  else schedule(std::false_type{});

  // ---- epilogue: OUT = O / l, LSE = (m + log2 l) ln 2
  const float lt = wave_sum_halves(w.l);
  const float inv = 1.0f / lt;
  if (qrow < a.Sq) {
    const int64_t orow = (row_base + qrow) * D;
#pragma unroll
    for (int db = 0; db < W::NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 val = {w.o[db][4 * j] * inv, w.o[db][4 * j + 1] * inv, w.o[db][4 * j + 2] * inv,
                           w.o[db][4 * j + 3] * inv};
        store_out4<OUT_BF16>(a.out, orow + db * 32 + 8 * j + 4 * half, val);
      }
    if (half == 0) lse[qrow] = (w.m + __log2f(lt)) * 0.69314718055994530942f;
  }
}

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
  const int64_t total = (int64_t)a.n_qtiles * a.B * a.H * a.P;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)total), block(kThreads);
  if (a.qk_fp8) {
    if (a.D == 128) {
      if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<128, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_bf16_kernel<128, false, true>), grid, block, 0, stream, a);
    } else if (a.D == 64) {
      if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<64, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_bf16_kernel<64, false, true>), grid, block, 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (a.D == 128) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<128, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, false, false>), grid, block, 0, stream, a);
  } else if (a.D == 64) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_bf16_kernel<64, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, false, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t gy = (int64_t)a.B * a.H * a.P;
  if (gy <= 0 || a.Sq <= 0) return hipSuccess;
  if (gy > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((a.Sq + kF32Rows - 1) / kF32Rows), (unsigned)gy), block(kF32Threads);
  const int dc = a.D / 4;
  if (dc <= 8) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_f32_kernel<8, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<8, false>), grid, block, 0, stream, a);
  } else if (dc <= 16) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_f32_kernel<16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<16, false>), grid, block, 0, stream, a);
  } else if (dc <= 32) {
    if (a.out_bf16) hipLaunchKernelGGL((attn_f32_kernel<32, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_f32_kernel<32, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace as
