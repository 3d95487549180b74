// Partition attention on CDNA4 (gfx950): per query row and per KV partition i,
// the attention state AS(i) = (OUT(i), LSE(i)) of exact softmax attention
// restricted to the keys of partition i.
//   DiTango review page (pith.science), "What carries the argument": the state of a
//   partition is its partial attention output with the log-sum-exp of its scores.
//
// bf16 kernel design (one workgroup = 8 waves = 256 query rows x one (batch, head)
// x one partition; one wave = 32 query rows; two waves per SIMD so that one
// wave's softmax overlaps the other's MFMA work):
//   * The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (M = 32 keys, N = 32 queries, K = 16 of D). In that accumulator layout a lane
//     holds 16 keys of ONE query row, so the row max needs one cross-half swap
//     (v_permlane32_swap) and the row sum stays lane-local until the epilogue.
//   * The accumulator registers of S^T are, key for key, the B operand of
//     O^T = V^T P^T (M = 32 of D, N = 32 queries, K = 16 keys) once rounded to bf16:
//     P never leaves registers.
//   * Q stays in registers for the whole partition. K tiles are staged in LDS as
//     [key][d] with 16-byte chunks XOR-swizzled by row; V tiles are transposed on
//     their way into LDS ([d][key], 4-key groups XOR-swizzled by d) so the V^T
//     operand is two 8-byte LDS reads per lane. Both are double buffered: the
//     global loads of tile t+1 are in flight while tile t is computed.
//   * Online softmax in the exp2 domain with a lazy rescale: the running max is
//     only moved (and O, l rescaled) when a new score exceeds it by more than
//     2^8, which is exact because the same max is used for O and l.
//   * Workgroups sharing a (batch, head, partition) are mapped to the same XCD so
//     that its L2 serves their common K/V tiles.
#include <hip/hip_runtime.h>
#include <math.h>

#include "as_internal.h"

namespace as {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kQB = 1;                       // 32-row query blocks per wave
constexpr int kRowsPerWave = 32 * kQB;       // 32
constexpr int kBQ = kWaves * kRowsPerWave;   // 256 query rows per workgroup
constexpr int kBK = 64;                      // keys per tile
constexpr int kThreads = kWaves * 64;
constexpr float kRescaleThreshold = 8.0f;    // log2 units

// Maps the hardware workgroup id to a logical tile id so that consecutive logical
// ids land on the same XCD (workgroups are dealt round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int x = L % kXcd, idx = L / kXcd;
  return (x < rem) ? x * (per + 1) + idx : rem * (per + 1) + (x - rem) * per + idx;
}

// Swizzle of the 8-byte (4-key) groups in a row d of the transposed V tile:
// conflict-free both for the staging writes (16 lanes on rows 8c+d') and for the
// operand reads (16 lanes on 16 consecutive rows).
__device__ __forceinline__ int vt_swz(int d) {
  return ((((d & 7) ^ ((d >> 4) & 7)) << 1) | ((d >> 3) & 1));
}

__device__ __forceinline__ float swap_halves(float x) {
  // v_permlane32_swap: returns {lanes 0-31 of x in the upper half, 32-63 in the lower}
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnArgs a) {
  constexpr int NDS = D / 16;        // MFMA k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int KTILE = kBK * D * 2; // bytes of one K tile
  constexpr int VTILE = D * kBK * 2; // bytes of one transposed V tile
  constexpr int STAGE = KTILE + VTILE;
  constexpr int KLOADS = kBK * KCH / kThreads;   // 16-byte K chunks per thread
  constexpr int VUNITS = (kBK / 4) * KCH;        // 4 keys x 8 d units of V
  static_assert(KLOADS >= 1 && VUNITS <= kThreads, "tile shape");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

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

  const int ks = a.ranges[2 * part], ke = a.ranges[2 * part + 1];
  const int n = ke - ks;
  const int q0 = qtile * kBQ;
  const int64_t row_base = ((int64_t)part * a.B * a.H + bh) * a.Sq;   // row index in out/lse
  float* __restrict__ out = a.out + row_base * D;
  float* __restrict__ lse = a.lse + row_base;

  if (n <= 0) {  // empty partition: the identity state (0, -inf)
    for (int r = tid; r < kBQ; r += kThreads) {
      const int q = q0 + r;
      if (q < a.Sq) {
        lse[q] = -INFINITY;
        f32x4* o4 = reinterpret_cast<f32x4*>(out + (int64_t)q * D);
        for (int c = 0; c < D / 4; ++c) o4[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  // ---- Q fragments (B operand of S^T): lane holds Q[row = l32][d = ds*16 + 8*half .. +7]
  const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb + hh * a.q_sh;
  bf16x8 qf[kQB][NDS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int q = q0 + wave * kRowsPerWave + qb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (q < a.Sq) x = *reinterpret_cast<const u32x4*>(qp + (int64_t)q * a.q_ss + ds * 16 + 8 * half);
      qf[qb][ds] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + b * a.k_sb + hh * a.k_sh + (int64_t)ks * a.k_ss;
  const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + b * a.k_sb + hh * a.k_sh + (int64_t)ks * a.k_ss;
  const int64_t kss = a.k_ss;
  const int ntiles = (n + kBK - 1) / kBK;

  // ---- staging registers and their LDS destinations
  u32x4 kreg[KLOADS];
  u32x4 vreg[4];
  const int vu_c = tid % KCH;       // V unit: 8-wide d chunk
  const int vu_a = tid / KCH;       // V unit: 4-key group
  const bool vu_on = tid < VUNITS;

  auto gload = [&](int tile) {
    const int key0 = tile * kBK;
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / KCH, ch = c % KCH;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key0 + row < n) x = *reinterpret_cast<const u32x4*>(kp + (int64_t)(key0 + row) * kss + ch * 8);
      kreg[j] = x;
    }
    if (vu_on) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * vu_a + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key0 + row < n) x = *reinterpret_cast<const u32x4*>(vp + (int64_t)(key0 + row) * kss + vu_c * 8);
        vreg[j] = x;
      }
    }
  };

  auto swrite = [&](int stage) {
    char* kt = smem + stage * STAGE;
#pragma unroll
    for (int j = 0; j < KLOADS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / KCH, ch = c % KCH;
      *reinterpret_cast<u32x4*>(kt + row * (D * 2) + ((ch ^ (row & (KCH - 1))) * 16)) = kreg[j];
    }
    if (vu_on) {
      char* vt = kt + KTILE;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned v0 = vreg[0][w], v1 = vreg[1][w], v2 = vreg[2][w], v3 = vreg[3][w];
        // d = 8c + 2w takes the low halves, d = 8c + 2w + 1 the high halves
        const u32x2 lo = {__builtin_amdgcn_perm(v1, v0, 0x05040100u), __builtin_amdgcn_perm(v3, v2, 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(v1, v0, 0x07060302u), __builtin_amdgcn_perm(v3, v2, 0x07060302u)};
        const int d0 = 8 * vu_c + 2 * w, d1 = d0 + 1;
        *reinterpret_cast<u32x2*>(vt + d0 * (kBK * 2) + ((vu_a ^ vt_swz(d0)) * 8)) = lo;
        *reinterpret_cast<u32x2*>(vt + d1 * (kBK * 2) + ((vu_a ^ vt_swz(d1)) * 8)) = hi;
      }
    }
  };

  // per-lane LDS read offsets
  const int krow_swz = l32 & (KCH - 1);
  int vt_off[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) vt_off[db] = (db * 32 + l32) * (kBK * 2);
  int vt_sw[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) vt_sw[db] = vt_swz(db * 32 + l32);

  f32x16 o[NDB][kQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) o[db][qb] = f32x16{};
  float m[kQB], l[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) { m[qb] = -INFINITY; l[qb] = 0.f; }
  const float c2 = a.scale_log2;

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const char* kt = smem + stage * STAGE;
    const char* vt = kt + KTILE;

    // ---- S^T = K Q^T : s[kb][qb], lane (l32, half), reg r <-> key kb*32 + 8(r/4) + 4half + r%4, query l32
    f32x16 s[2][kQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int row = kb * 32 + l32;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + row * (D * 2) + (((2 * ds + half) ^ krow_swz) * 16));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }

    // ---- mask keys past the end of the partition (last tile only)
    const int valid = n - t * kBK;
    if (valid < kBK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= valid) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[kb][qb][r] = -INFINITY;
          }
        }
    }

    // ---- online softmax (exp2 domain, lazy rescale)
    float mx[kQB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float x = s[0][qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, s[0][qb][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, s[1][qb][r]);
      mx[qb] = wave_max_halves(x) * c2;
      need |= mx[qb] > m[qb] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float mn = fmaxf(m[qb], mx[qb]);
        const float f = __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
        l[qb] *= f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][qb] *= f;
      }
    }
    bf16x8 pf[kQB][2][2];   // [qb][kb][c]: B operand of O^T for keys kb*32 + 16c + ...
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float nm = -m[qb];
      // the row sum uses the fp32 probabilities: summing their bf16 roundings
      // would put the bf16 unit roundoff (2^-8) straight into LSE
      float acc0 = l[qb], acc1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8 p;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * c + e], c2, nm));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * c + e + 1], c2, nm));
            acc0 += p0;
            acc1 += p1;
            p[e] = (__bf16)p0;
            p[e + 1] = (__bf16)p1;
          }
          pf[qb][kb][c] = p;
        }
      l[qb] = acc0 + acc1;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int g = 8 * kb + 4 * c + half;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vt + vt_off[db] + ((g ^ vt_sw[db]) * 8));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + vt_off[db] + (((g + 2) ^ vt_sw[db]) * 8));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][c], o[db][qb], 0, 0, 0);
        }
      }

    if (t + 1 < ntiles) swrite(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: OUT = O / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float lt = wave_sum_halves(l[qb]);
    const float inv = 1.0f / lt;
    const int q = q0 + wave * kRowsPerWave + qb * 32 + l32;
    if (q < a.Sq) {
      float* orow = out + (int64_t)q * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 val = {o[db][qb][4 * j] * inv, o[db][qb][4 * j + 1] * inv,
                             o[db][qb][4 * j + 2] * inv, o[db][qb][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * j + 4 * half) = val;
        }
      if (half == 0) lse[q] = (m[qb] + __log2f(lt)) * 0.69314718055994530942f;
    }
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

template <int DC>  // D / 4 elements per lane (1..32)
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
  float* out = a.out + row_base * D;
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
      for (int e = 0; e < dc; ++e) out[(int64_t)q * D + sub * dc + e] = 0.f;
      if (sub == 0) lse[q] = -INFINITY;
    } else {
      for (int e = 0; e < DC; ++e)
        if (e < dc) out[(int64_t)q * D + sub * dc + e] = acc[e] / l;
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
  if (a.D == 128) {
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, stream, a);
  } else if (a.D == 64) {
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, stream, a);
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
    hipLaunchKernelGGL(attn_f32_kernel<8>, grid, block, 0, stream, a);
  } else if (dc <= 16) {
    hipLaunchKernelGGL(attn_f32_kernel<16>, grid, block, 0, stream, a);
  } else if (dc <= 32) {
    hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace as
