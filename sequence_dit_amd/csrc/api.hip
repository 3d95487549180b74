// C ABI of the attention-state library: host-side validation, argument packing and
// launches on the caller's stream. Every check runs before the first HIP call, so
// invalid arguments never reach the device; nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "as_internal.h"

namespace {

thread_local char g_last_error[512] = "";

as_status fail(as_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

as_status ok() {
  g_last_error[0] = '\0';
  return AS_OK;
}

as_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(AS_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) share at least one byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Product of non-negative sizes, or -1 when it does not fit in int64.
int64_t mul3(int64_t a, int64_t b, int64_t c = 1) {
  int64_t r;
  if (__builtin_mul_overflow(a, b, &r) || __builtin_mul_overflow(r, c, &r)) return -1;
  return r;
}

// Bytes from the first to one past the last element of a [n0][n1][n2][D] tensor with
// element strides s[0..2] (unit stride on the last dimension), or -1 on overflow.
// Every n >= 1.
int64_t extent_bytes(int64_t n0, int64_t n1, int64_t n2, int64_t D, const int64_t s[3], int64_t esz) {
  int64_t t0, t1, t2, r;
  if (__builtin_mul_overflow(n0 - 1, s[0], &t0) || __builtin_mul_overflow(n1 - 1, s[1], &t1) ||
      __builtin_mul_overflow(n2 - 1, s[2], &t2) || __builtin_add_overflow(t0, t1, &r) ||
      __builtin_add_overflow(r, t2, &r) || __builtin_add_overflow(r, D, &r) || __builtin_mul_overflow(r, esz, &r))
    return -1;
  return r;
}

// Sizes accepted for a state block (rows * D elements): far beyond any device memory,
// small enough that byte counts never overflow.
constexpr int64_t kMaxRows = (int64_t)1 << 40;

// Storage kind of a state dtype, or -1.
int out_kind(as_dtype t) {
  return t == AS_F32 ? as::kOutF32 : t == AS_BF16 ? as::kOutBF16 : t == AS_FP8_E4M3 ? as::kOutFP8 : -1;
}

// Bytes of one state's OUT of `rows` rows (rows * D <= kMaxRows * 1024 by the callers).
int64_t state_bytes(as_dtype t, int64_t rows, int64_t D) {
  return t == AS_FP8_E4M3 ? as::fp8_payload_bytes(rows, D) : rows * D * (t == AS_BF16 ? 2 : 4);
}

}  // namespace

extern "C" {

const char* as_status_string(as_status s) {
  switch (s) {
    case AS_OK: return "ok";
    case AS_ERR_INVALID_ARG: return "invalid argument";
    case AS_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case AS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* as_last_error(void) { return g_last_error; }

namespace {

// Grid of a grouped launch: (G * B * H units rounded up to a multiple of 8) * query tiles.
as_status check_grid_grouped(int32_t G, int64_t B, int64_t H, int64_t Sq, int64_t D) {
  const int64_t bq = as::attn_bf16_rows_per_block((int)D);
  const int64_t units = ((int64_t)G * B * H + 7) / 8 * 8;
  if (units * ((Sq + bq - 1) / bq) > 0x7fffffff) return fail(AS_ERR_UNSUPPORTED, "grid too large");
  return AS_OK;
}

// The grouped variant's extra arguments (as_partition_attn_grouped).
struct Grouping {
  const int32_t* starts;
  int32_t G;
  const float* fold_out;
  const float* fold_lse;
  float* part_lse;
};

as_status attn_impl(const void* q, const void* k, const void* v, as_dtype dtype,
                    int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                    const int64_t q_stride[3], const int64_t kv_stride[3],
                    const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                    void* out, float* lse, hipStream_t stream,
                    bool qk_fp8 = false, const float* q_scale = nullptr, const float* k_scale = nullptr,
                    const Grouping* grouping = nullptr, bool v_fp8 = false, const float* v_scale = nullptr) {
  if (dtype != AS_BF16 && dtype != AS_F32) return fail(AS_ERR_INVALID_ARG, "dtype %d is not AS_BF16 or AS_F32", (int)dtype);
  if (out_kind(state_dtype) < 0)
    return fail(AS_ERR_INVALID_ARG, "state_dtype %d is not AS_F32, AS_BF16 or AS_FP8_E4M3", (int)state_dtype);
  if (state_dtype == AS_FP8_E4M3 && dtype == AS_F32)
    return fail(AS_ERR_UNSUPPORTED, "the f32 path writes AS_F32 or AS_BF16 states");
  if (B < 0 || H < 0 || Sq < 0 || Skv < 0) return fail(AS_ERR_INVALID_ARG, "negative size (B=%lld H=%lld Sq=%lld Skv=%lld)",
                                                       (long long)B, (long long)H, (long long)Sq, (long long)Skv);
  if (D < 1) return fail(AS_ERR_INVALID_ARG, "D=%lld must be positive", (long long)D);
  if (P < 0 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [0, %d]", P, AS_MAX_PARTITIONS);
  if (!(isfinite(scale) && scale >= 0.f)) return fail(AS_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (P > 0 && !kv_ranges) return fail(AS_ERR_INVALID_ARG, "kv_ranges is NULL");
  for (int32_t i = 0; i < P; ++i) {
    const int64_t s = kv_ranges[2 * i], e = kv_ranges[2 * i + 1];
    if (s < 0 || e < s || e > Skv)
      return fail(AS_ERR_INVALID_ARG, "kv_ranges[%d] = [%lld, %lld) is not within [0, Skv=%lld] with start <= end",
                  i, (long long)s, (long long)e, (long long)Skv);
  }
  if (dtype == AS_BF16 && D != 64 && D != 128)
    return fail(AS_ERR_UNSUPPORTED, "%s path supports D in {64, 128}, got %lld", qk_fp8 ? "fp8" : "bf16", (long long)D);
  if (dtype == AS_F32 && (D % 4 != 0 || D > 128))
    return fail(AS_ERR_UNSUPPORTED, "f32 path supports D a multiple of 4 up to 128, got %lld", (long long)D);
  // outputs: P partition states, or G group states (grouped)
  int64_t n_states = P;
  if (grouping) {
    const Grouping& g = *grouping;
    if (P < 1) return fail(AS_ERR_INVALID_ARG, "grouped launches need P >= 1");
    if (g.G < 1 || g.G > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "G=%d outside [1, %d]", g.G, AS_MAX_PARTITIONS);
    if (!g.starts) return fail(AS_ERR_INVALID_ARG, "group_starts is NULL");
    if (g.starts[0] != 0 || g.starts[g.G] != P)
      return fail(AS_ERR_INVALID_ARG, "group_starts must run from 0 to P=%d", P);
    for (int32_t i = 0; i < g.G; ++i)
      if (g.starts[i + 1] < g.starts[i]) return fail(AS_ERR_INVALID_ARG, "group_starts decreases at %d", i);
    if ((g.fold_out == nullptr) != (g.fold_lse == nullptr))
      return fail(AS_ERR_INVALID_ARG, "fold_out and fold_lse must both be given or both be NULL");
    if (state_dtype != AS_F32) return fail(AS_ERR_INVALID_ARG, "grouped launches write float32 states");
    n_states = g.G;
  }
  if (B == 0 || H == 0 || Sq == 0 || P == 0) return ok();
  if (B > 65535 || H > 65535 || B * H > 65535) return fail(AS_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)mul3(B, H));
  if (Sq > 0x7fffffff || Skv > 0x7fffffff) return fail(AS_ERR_UNSUPPORTED, "sequence length exceeds 2^31-1");
  const int64_t rows = B * H * Sq;
  if (!q || !k || !v || !out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!q_stride || !kv_stride) return fail(AS_ERR_INVALID_ARG, "NULL stride array");
  if (qk_fp8 && (!q_scale || !k_scale)) return fail(AS_ERR_INVALID_ARG, "q_scale and k_scale must not be NULL");
  if (qk_fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4)))
    return fail(AS_ERR_INVALID_ARG, "q_scale and k_scale must be 4-byte aligned");
  if (v_fp8 && (!v_scale || !aligned(v_scale, 4))) return fail(AS_ERR_INVALID_ARG, "v_scale must be non-NULL and 4-byte aligned");
  // bytes per v element (the widest input)
  const int64_t esz = v_fp8 ? 1 : dtype == AS_BF16 ? 2 : 4;
  // fp8 rows are read 16 bytes at a time: 16 one-byte elements
  const int64_t smul = qk_fp8 ? 16 : dtype == AS_BF16 ? 8 : 4;
  for (int j = 0; j < 3; ++j) {
    if (q_stride[j] < 0 || kv_stride[j] < 0) return fail(AS_ERR_INVALID_ARG, "negative stride");
    if (q_stride[j] % smul || kv_stride[j] % smul)
      return fail(AS_ERR_INVALID_ARG, "strides must be multiples of %lld elements", (long long)smul);
  }
  if (q_stride[2] < D || kv_stride[2] < D) return fail(AS_ERR_INVALID_ARG, "sequence stride smaller than D");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return fail(AS_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  if (!aligned(out, 16) || !aligned(lse, 4)) return fail(AS_ERR_INVALID_ARG, "out must be 16-byte and lse 4-byte aligned");
  // The bf16/fp8 kernels address the rows of a key tile (up to 128 keys, also past a
  // shorter range's end) with 32-bit byte offsets from the tile's first row.
  for (int32_t i = 0; i < P; ++i) {
    const int64_t n = (int64_t)kv_ranges[2 * i + 1] - kv_ranges[2 * i];
    const int64_t span = mul3(n > 128 ? n : 128, kv_stride[2], esz);
    if (span < 0 || span >= ((int64_t)1 << 31))
      return fail(AS_ERR_UNSUPPORTED, "kv range %d spans 2^31 bytes or more", i);
  }
  // Outputs must not overlap each other or any byte an input may occupy.
  const int64_t qesz = qk_fp8 ? 1 : esz, kesz = qk_fp8 ? 1 : esz;
  const int64_t q_bytes = extent_bytes(B, H, Sq, D, q_stride, qesz);
  const int64_t k_bytes = Skv > 0 ? extent_bytes(B, H, Skv, D, kv_stride, kesz) : 0;
  const int64_t v_bytes = Skv > 0 ? extent_bytes(B, H, Skv, D, kv_stride, esz) : 0;
  const int64_t out_bytes = mul3(n_states, state_bytes(state_dtype, rows, D));
  const int64_t lse_bytes = mul3(n_states, rows, 4);
  if (q_bytes < 0 || k_bytes < 0 || v_bytes < 0 || out_bytes < 0 || lse_bytes < 0)
    return fail(AS_ERR_UNSUPPORTED, "tensor extents overflow 64-bit byte counts");
  if (overlap(out, (size_t)out_bytes, lse, (size_t)lse_bytes)) return fail(AS_ERR_INVALID_ARG, "out and lse overlap");
  const void* ins[8] = {q, k, v, nullptr, nullptr, q_scale, k_scale, v_scale};
  const int64_t sbytes = qk_fp8 ? B * H * 4 : 0;
  int64_t in_bytes[8] = {q_bytes, k_bytes, v_bytes, 0, 0, sbytes, sbytes, v_fp8 ? B * H * 4 : 0};
  const float* part_lse = nullptr;
  const size_t part_bytes = (size_t)(P * rows) * 4;
  if (grouping) {
    const Grouping& g = *grouping;
    if (g.fold_out && (!aligned(g.fold_out, 16) || !aligned(g.fold_lse, 4)))
      return fail(AS_ERR_INVALID_ARG, "fold_out must be 16-byte and fold_lse 4-byte aligned");
    if (g.part_lse && !aligned(g.part_lse, 4)) return fail(AS_ERR_INVALID_ARG, "part_lse must be 4-byte aligned");
    ins[3] = g.fold_out;
    in_bytes[3] = rows * D * 4;
    ins[4] = g.fold_lse;
    in_bytes[4] = rows * 4;
    part_lse = g.part_lse;
    if (overlap(part_lse, part_bytes, out, (size_t)out_bytes) || overlap(part_lse, part_bytes, lse, (size_t)lse_bytes))
      return fail(AS_ERR_INVALID_ARG, "part_lse overlaps out or lse");
  }
  static const char* const in_names[8] = {"q", "k", "v", "fold_out", "fold_lse", "q_scale", "k_scale", "v_scale"};
  for (int j = 0; j < 8; ++j)
    if (overlap(out, (size_t)out_bytes, ins[j], (size_t)in_bytes[j]) ||
        overlap(lse, (size_t)lse_bytes, ins[j], (size_t)in_bytes[j]) ||
        overlap(part_lse, part_bytes, ins[j], (size_t)in_bytes[j]))
      return fail(AS_ERR_INVALID_ARG, "an output overlaps input %s", in_names[j]);

  as::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v;
  a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_ss = q_stride[2];
  a.k_sb = kv_stride[0]; a.k_sh = kv_stride[1]; a.k_ss = kv_stride[2];
  a.out = out; a.lse = lse;
  a.out_kind = out_kind(state_dtype);
  a.qk_fp8 = qk_fp8 ? 1 : 0;
  a.v_fp8 = v_fp8 ? 1 : 0;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.state_rows = rows;
  a.payload_bytes = state_dtype == AS_FP8_E4M3 ? as::fp8_payload_bytes(rows, D) : 0;
  a.B = (int32_t)B; a.H = (int32_t)H; a.Sq = (int32_t)Sq; a.Skv = (int32_t)Skv; a.D = (int32_t)D; a.P = P;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  for (int32_t i = 0; i < 2 * P; ++i) a.ranges[i] = kv_ranges[i];

  if (grouping) {
    // The kernel walks the non-empty partitions only: pack them in group order and keep
    // each one's index for its LSE; the LSE of an empty partition is -inf.
    const as_status gs = check_grid_grouped(grouping->G, B, H, Sq, D);
    if (gs != AS_OK) return gs;
    a.G = grouping->G;
    a.fold_out = grouping->fold_out;
    a.fold_lse = grouping->fold_lse;
    a.part_lse = grouping->part_lse;
    int32_t packed = 0;
    for (int32_t g = 0; g < grouping->G; ++g) {
      a.group_starts[g] = (uint16_t)packed;
      for (int32_t i = grouping->starts[g]; i < grouping->starts[g + 1]; ++i) {
        if (kv_ranges[2 * i + 1] > kv_ranges[2 * i]) {
          a.ranges[2 * packed] = kv_ranges[2 * i];
          a.ranges[2 * packed + 1] = kv_ranges[2 * i + 1];
          a.part_index[packed] = (uint16_t)i;
          ++packed;
        }
      }
    }
    a.group_starts[grouping->G] = (uint16_t)packed;
    for (int32_t i = packed; i < P; ++i) a.ranges[2 * i] = a.ranges[2 * i + 1] = 0;
    a.P = packed;
    const int bq = as::attn_bf16_rows_per_block((int)D);
    a.n_qtiles = (int32_t)((Sq + bq - 1) / bq);
    if (grouping->part_lse) {
      for (int32_t i = 0; i < P; ++i)
        if (kv_ranges[2 * i + 1] <= kv_ranges[2 * i]) {
          const hipError_t e = as::launch_fill_neg_inf(grouping->part_lse + (int64_t)i * rows, rows, stream);
          if (e != hipSuccess) return hip_status(e, "partition_attn grouped: empty partition LSE");
        }
    }
    return hip_status(as::launch_attn_grouped(a, stream), "partition_attn grouped launch");
  }
  if (dtype == AS_BF16) {
    const int bq = as::attn_bf16_rows_per_block((int)D);
    a.n_qtiles = (int32_t)((Sq + bq - 1) / bq);
    if ((B * H * P + 7) / 8 * 8 * a.n_qtiles > 0x7fffffff) return fail(AS_ERR_UNSUPPORTED, "grid too large");
    return hip_status(as::launch_attn_bf16(a, stream), "partition_attn bf16 launch");
  }
  const int bq = as::attn_f32_rows_per_block((int)D);
  a.n_qtiles = (int32_t)((Sq + bq - 1) / bq);
  if (B * H * P > 65535) return fail(AS_ERR_UNSUPPORTED, "f32 path: B*H*P=%lld exceeds 65535", (long long)(B * H * P));
  return hip_status(as::launch_attn_f32(a, stream), "partition_attn f32 launch");
}

// Checks shared by the composition calls: state dtypes and D.
as_status check_state_types(as_dtype in_dtype, as_dtype out_dtype, int64_t D) {
  if (out_kind(in_dtype) < 0 || out_kind(out_dtype) < 0)
    return fail(AS_ERR_INVALID_ARG, "state dtypes must be AS_F32, AS_BF16 or AS_FP8_E4M3");
  if (D < 4 || D > 1024 || D % 4) return fail(AS_ERR_INVALID_ARG, "D=%lld must be a multiple of 4 in [4, 1024]", (long long)D);
  if ((in_dtype == AS_FP8_E4M3 || out_dtype == AS_FP8_E4M3) && D != 32 && D != 64 && D != 128 && D != 256)
    return fail(AS_ERR_UNSUPPORTED, "fp8 states need D in {32, 64, 128, 256}, got %lld", (long long)D);
  return AS_OK;
}

// Alignment of a state's OUT pointer: 16 bytes (fp32, fp8 payloads), 8 (bf16).
size_t state_align(as_dtype t) { return t == AS_BF16 ? 8 : 16; }

as_status merge_impl(int32_t n, const void* const* outs, const float* const* lses, as_dtype in_dtype,
                     int64_t rows, int64_t D, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  const as_status ts = check_state_types(in_dtype, out_dtype, D);
  if (ts != AS_OK) return ts;
  if (n < 1 || n > AS_MAX_MERGE) return fail(AS_ERR_INVALID_ARG, "n=%d outside [1, %d]", n, AS_MAX_MERGE);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (!outs || !lses) return fail(AS_ERR_INVALID_ARG, "NULL pointer list");
  if (rows == 0) return ok();
  if (rows > kMaxRows) return fail(AS_ERR_UNSUPPORTED, "rows=%lld too large", (long long)rows);
  if (!out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL output pointer");
  // OUT is read and written 4 elements at a time: 16 bytes of fp32, 8 of bf16; fp8
  // payloads up to 16 codes at a time
  const size_t ain = state_align(in_dtype), aout = state_align(out_dtype);
  if (!aligned(out, aout) || !aligned(lse, 4))
    return fail(AS_ERR_INVALID_ARG, "out must be %zu-byte and lse 4-byte aligned", aout);
  const size_t in_bytes = (size_t)state_bytes(in_dtype, rows, D);
  const size_t out_bytes = (size_t)state_bytes(out_dtype, rows, D);
  const size_t lse_bytes = (size_t)rows * 4;
  if (overlap(out, out_bytes, lse, lse_bytes)) return fail(AS_ERR_INVALID_ARG, "out and lse overlap");
  as::MergeArgs a;
  memset(&a, 0, sizeof(a));
  for (int32_t i = 0; i < n; ++i) {
    if (!outs[i] || !lses[i]) return fail(AS_ERR_INVALID_ARG, "input %d has a NULL pointer", i);
    if (!aligned(outs[i], ain) || !aligned(lses[i], 4)) return fail(AS_ERR_INVALID_ARG, "input %d is misaligned", i);
    if (overlap(outs[i], in_bytes, out, out_bytes) || overlap(outs[i], in_bytes, lse, lse_bytes) ||
        overlap(lses[i], lse_bytes, out, out_bytes) || overlap(lses[i], lse_bytes, lse, lse_bytes))
      return fail(AS_ERR_INVALID_ARG, "input %d overlaps the output", i);
    a.outs[i] = outs[i];
    a.lses[i] = lses[i];
  }
  a.out = out; a.lse = lse; a.rows = rows; a.n = n; a.D = (int32_t)D;
  a.in_kind = out_kind(in_dtype); a.out_kind = out_kind(out_dtype);
  a.payload_bytes = as::fp8_payload_bytes(rows, D);
  a.vec2 = D % 8 == 0 && aligned(out, 16);
  for (int32_t i = 0; i < n; ++i) a.vec2 = a.vec2 && aligned(outs[i], 16);
  return hip_status(as::launch_merge(a, stream), "merge launch");
}

}  // namespace

as_status as_partition_attn(const void* q, const void* k, const void* v, as_dtype dtype,
                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                            const int64_t q_stride[3], const int64_t kv_stride[3],
                            const int32_t* kv_ranges, int32_t P, float scale,
                            float* out, float* lse, hipStream_t stream) {
  return attn_impl(q, k, v, dtype, B, H, Sq, Skv, D, q_stride, kv_stride, kv_ranges, P, scale, AS_F32, out, lse,
                   stream);
}

as_status as_partition_attn_states(const void* q, const void* k, const void* v, as_dtype dtype,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                   const int64_t q_stride[3], const int64_t kv_stride[3],
                                   const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                   void* out, float* lse, hipStream_t stream) {
  return attn_impl(q, k, v, dtype, B, H, Sq, Skv, D, q_stride, kv_stride, kv_ranges, P, scale, state_dtype, out, lse,
                   stream);
}

as_status as_partition_attn_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                const float* k_scale, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                const int64_t q_stride[3], const int64_t kv_stride[3],
                                const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                void* out, float* lse, hipStream_t stream) {
  return attn_impl(q, k, v, AS_BF16, B, H, Sq, Skv, D, q_stride, kv_stride, kv_ranges, P, scale, state_dtype, out, lse,
                   stream, true, q_scale, k_scale);
}

as_status as_partition_attn_fp8_qkv(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int64_t B, int64_t H, int64_t Sq,
                                    int64_t Skv, int64_t D, const int64_t q_stride[3], const int64_t kv_stride[3],
                                    const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                    void* out, float* lse, hipStream_t stream) {
  return attn_impl(q, k, v, AS_BF16, B, H, Sq, Skv, D, q_stride, kv_stride, kv_ranges, P, scale, state_dtype, out, lse,
                   stream, true, q_scale, k_scale, nullptr, true, v_scale);
}

as_status as_partition_attn_grouped(const void* q, const void* k, const void* v, as_dtype dtype,
                                    const float* q_scale, const float* k_scale, const float* v_scale, int64_t B, int64_t H,
                                    int64_t Sq, int64_t Skv, int64_t D, const int64_t q_stride[3],
                                    const int64_t kv_stride[3], const int32_t* kv_ranges, int32_t P,
                                    const int32_t* group_starts, int32_t G, float scale, const float* fold_out,
                                    const float* fold_lse, float* out, float* lse, float* part_lse,
                                    hipStream_t stream) {
  if (dtype != AS_BF16 && dtype != AS_FP8_E4M3)
    return fail(AS_ERR_INVALID_ARG, "dtype %d is not AS_BF16 or AS_FP8_E4M3", (int)dtype);
  const Grouping g = {group_starts, G, fold_out, fold_lse, part_lse};
  const bool fp8 = dtype == AS_FP8_E4M3, v8 = fp8 && v_scale != nullptr;
  return attn_impl(q, k, v, AS_BF16, B, H, Sq, Skv, D, q_stride, kv_stride, kv_ranges, P, scale, AS_F32, out, lse,
                   stream, fp8, fp8 ? q_scale : nullptr, fp8 ? k_scale : nullptr, &g, v8, v8 ? v_scale : nullptr);
}

as_status as_merge_states(int32_t n, const void* const* outs, const float* const* lses, as_dtype in_dtype,
                          int64_t rows, int64_t D, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  return merge_impl(n, outs, lses, in_dtype, rows, D, out_dtype, out, lse, stream);
}

as_status as_compose_groups(const void* outs, const float* lses, as_dtype in_dtype, int32_t P, int64_t rows,
                            int64_t D, int32_t group, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  const as_status ts = check_state_types(in_dtype, out_dtype, D);
  if (ts != AS_OK) return ts;
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (group < 1 || group > AS_MAX_MERGE) return fail(AS_ERR_INVALID_ARG, "group=%d outside [1, %d]", group, AS_MAX_MERGE);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (rows == 0) return ok();
  if (rows > kMaxRows) return fail(AS_ERR_UNSUPPORTED, "rows=%lld too large", (long long)rows);
  if (!outs || !lses || !out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(outs, 16) || !aligned(out, 16) || !aligned(lses, 4) || !aligned(lse, 4))
    return fail(AS_ERR_INVALID_ARG, "OUT blocks must be 16-byte and LSE blocks 4-byte aligned");
  const int64_t G = (P + group - 1) / group;
  const size_t in_block = (size_t)(P * state_bytes(in_dtype, rows, D));
  const size_t out_block = (size_t)(G * state_bytes(out_dtype, rows, D));
  if (overlap(outs, in_block, out, out_block) || overlap(lses, (size_t)(P * rows) * 4, lse, (size_t)(G * rows) * 4) ||
      overlap(outs, in_block, lse, (size_t)(G * rows) * 4) || overlap(lses, (size_t)(P * rows) * 4, out, out_block))
    return fail(AS_ERR_INVALID_ARG, "outputs overlap the input blocks");
  if (overlap(out, out_block, lse, (size_t)(G * rows) * 4)) return fail(AS_ERR_INVALID_ARG, "out and lse overlap");
  as::MergeArgs a;
  memset(&a, 0, sizeof(a));
  a.base_out = outs; a.base_lse = lses; a.out = out; a.lse = lse;
  a.rows = rows; a.n = P; a.D = (int32_t)D; a.group = group;
  a.in_kind = out_kind(in_dtype); a.out_kind = out_kind(out_dtype);
  a.payload_bytes = as::fp8_payload_bytes(rows, D);
  a.vec2 = D % 8 == 0;   // slices of rows*D elements keep 16-byte alignment when D % 8 == 0
  return hip_status(as::launch_merge(a, stream), "compose_groups launch");
}

as_status as_merge(int32_t n, const float* const* outs, const float* const* lses,
                   int64_t rows, int64_t D, float* out, float* lse, hipStream_t stream) {
  const void* ptrs[AS_MAX_MERGE];
  if (n >= 1 && n <= AS_MAX_MERGE && outs)
    for (int32_t i = 0; i < n; ++i) ptrs[i] = outs[i];
  return merge_impl(n, (n >= 1 && n <= AS_MAX_MERGE && outs) ? ptrs : nullptr, lses, AS_F32, rows, D, AS_F32, out, lse,
                    stream);
}

size_t as_state_bytes(as_dtype state_dtype, int64_t rows, int64_t D) {
  if (out_kind(state_dtype) < 0 || rows < 0 || rows > kMaxRows || D < 1 || D > 1024) return 0;
  return (size_t)state_bytes(state_dtype, rows, D);
}

size_t as_partition_contribution_workspace_size(int32_t P, int64_t rows, int64_t rows_per_group) {
  if (P < 1 || P > AS_MAX_PARTITIONS || rows < 0 || rows > kMaxRows || rows_per_group < 1 || rows % rows_per_group)
    return 0;
  const int64_t G = rows / rows_per_group;
  const int64_t chunks = (rows_per_group + as::kContribChunk - 1) / as::kContribChunk;
  return (size_t)(G * chunks * P) * sizeof(float);
}

namespace {
// Shared by as_partition_contribution (caller workspace) and
// as_partition_contribution_noalloc (library scratch, noalloc = true).
as_status contribution_impl(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group, float* weights,
                            float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            bool noalloc) {
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (rows_per_group < 1) return fail(AS_ERR_INVALID_ARG, "rows_per_group=%lld must be >= 1", (long long)rows_per_group);
  if (rows % rows_per_group) return fail(AS_ERR_INVALID_ARG, "rows=%lld is not a multiple of rows_per_group=%lld",
                                         (long long)rows, (long long)rows_per_group);
  if (rows == 0 || (!weights && !scores)) return ok();
  if (!lse) return fail(AS_ERR_INVALID_ARG, "lse is NULL");
  if (!aligned(lse, 4) || (weights && !aligned(weights, 4)) || (scores && !aligned(scores, 4)))
    return fail(AS_ERR_INVALID_ARG, "misaligned pointer");
  if (rows > kMaxRows || (int64_t)P * rows > kMaxRows) return fail(AS_ERR_UNSUPPORTED, "P*rows too large");
  const size_t need = as_partition_contribution_workspace_size(P, rows, rows_per_group);
  if (noalloc && scores && need > as::kContribScratchBytes)
    return fail(AS_ERR_INVALID_ARG, "scores of these sizes need %zu bytes of scratch; the library holds %zu",
                need, as::kContribScratchBytes);
  if (scores && !noalloc) {
    if (!workspace) return fail(AS_ERR_INVALID_ARG, "workspace is NULL but scores were requested");
    if (workspace_bytes < need)
      return fail(AS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(AS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  {
    const size_t lb = (size_t)(P * rows) * 4, wb = weights ? lb : 0;
    const size_t sb = scores ? (size_t)((rows / rows_per_group) * P) * 4 : 0, kb = scores && !noalloc ? need : 0;
    if (overlap(weights, wb, lse, lb) || overlap(scores, sb, lse, lb) || overlap(workspace, kb, lse, lb) ||
        overlap(weights, wb, scores, sb) || overlap(weights, wb, workspace, kb) || overlap(scores, sb, workspace, kb))
      return fail(AS_ERR_INVALID_ARG, "weights, scores, workspace and lse must not overlap");
  }
  float* partial = nullptr;
  if (scores && noalloc) {
    const hipError_t e = as::contribution_scratch(&partial);
    if (e != hipSuccess) return hip_status(e, "scratch address lookup");
  } else if (scores) {
    partial = static_cast<float*>(workspace);
  }
  as::ContribArgs a;
  memset(&a, 0, sizeof(a));
  a.lse = lse; a.weights = weights; a.scores = scores;
  a.partial = partial;
  a.rows = rows; a.rows_per_group = rows_per_group; a.P = P;
  a.chunks_per_group = (int32_t)((rows_per_group + as::kContribChunk - 1) / as::kContribChunk);
  return hip_status(as::launch_contribution(a, stream), "partition_contribution launch");
}
}  // namespace

as_status as_partition_contribution(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group,
                                    float* weights, float* scores, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return contribution_impl(lse, P, rows, rows_per_group, weights, scores, workspace, workspace_bytes, stream, false);
}

as_status as_partition_contribution_noalloc(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group,
                                            float* weights, float* scores, hipStream_t stream) {
  return contribution_impl(lse, P, rows, rows_per_group, weights, scores, nullptr, 0, stream, true);
}


size_t as_state_norms_workspace_size(int32_t P, int64_t n) {
  if (P < 1 || P > AS_MAX_PARTITIONS || n < 0 || n % 4 || n > ((int64_t)1 << 40)) return 0;
  return (size_t)(P * as::norms_chunks(P, n)) * sizeof(double);
}

as_status as_state_norms(const float* a, const float* b, int32_t P, int64_t n, float* norms,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (n < 0 || n % 4) return fail(AS_ERR_INVALID_ARG, "n=%lld must be a non-negative multiple of 4", (long long)n);
  if (n > ((int64_t)1 << 40)) return fail(AS_ERR_UNSUPPORTED, "n=%lld too large", (long long)n);
  if (!norms) return fail(AS_ERR_INVALID_ARG, "norms is NULL");
  if (n > 0 && !a) return fail(AS_ERR_INVALID_ARG, "a is NULL");
  if (!aligned(a, 16) || !aligned(b, 16)) return fail(AS_ERR_INVALID_ARG, "a and b must be 16-byte aligned");
  if (!aligned(norms, 4)) return fail(AS_ERR_INVALID_ARG, "misaligned norms");
  const size_t need = as_state_norms_workspace_size(P, n);
  if (!workspace) return fail(AS_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(AS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(AS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  {
    const size_t ib = (size_t)(P * n) * 4, nb = (size_t)P * 4;
    const void* bb = n > 0 ? b : nullptr;
    if (overlap(norms, nb, a, ib) || overlap(norms, nb, bb, ib) || overlap(workspace, need, a, ib) ||
        overlap(workspace, need, bb, ib) || overlap(workspace, need, norms, nb))
      return fail(AS_ERR_INVALID_ARG, "norms, workspace and the inputs must not overlap");
  }
  as::NormArgs g;
  memset(&g, 0, sizeof(g));
  g.a = a; g.b = (n > 0) ? b : nullptr; g.norms = norms; g.partial = static_cast<double*>(workspace);
  g.n = n; g.chunk = as::norms_chunk(P, n); g.P = P; g.chunks = (int32_t)as::norms_chunks(P, n);
  return hip_status(as::launch_state_norms(g, stream), "state_norms launch");
}

namespace {
as_status check_groups(int32_t P, int32_t local, int32_t group) {
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (local < 0 || local >= P) return fail(AS_ERR_INVALID_ARG, "local=%d outside [0, P=%d)", local, P);
  if (group < 1) return fail(AS_ERR_INVALID_ARG, "group=%d must be >= 1", group);
  return AS_OK;
}
}  // namespace

as_status as_planner_decide(const float* anchor_norms, const float* local_drift, const float* weights,
                            const float* eps, int32_t P, int32_t local, int32_t group, float eps_local,
                            float* alpha, float* delta, float* ase, int32_t* compute, int32_t* anchor,
                            hipStream_t stream) {
  const as_status st = check_groups(P, local, group);
  if (st != AS_OK) return st;
  if (!isfinite(eps_local)) return fail(AS_ERR_INVALID_ARG, "eps_local must be finite");
  if (!anchor_norms || !local_drift || !weights || !eps || !compute || !anchor)
    return fail(AS_ERR_INVALID_ARG, "anchor_norms, local_drift, weights, eps, compute and anchor must not be NULL");
  const void* ptrs[] = {anchor_norms, local_drift, weights, eps, alpha, delta, ase, compute, anchor};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return fail(AS_ERR_INVALID_ARG, "misaligned pointer");
  {
    const int32_t ge = group > P ? P : group;
    const size_t G = (size_t)((P + ge - 1) / ge);
    const void* ip[] = {anchor_norms, local_drift, weights, eps};
    const size_t ib[] = {(size_t)P * 4, 4, (size_t)P * 4, 4};
    const void* op[] = {alpha, delta, ase, compute, anchor};
    const size_t ob[] = {(size_t)P * 4, (size_t)P * 4, G * 4, G * 4, 4};
    for (int o = 0; o < 5; ++o) {
      for (int i = 0; i < 4; ++i)
        if (overlap(op[o], ob[o], ip[i], ib[i])) return fail(AS_ERR_INVALID_ARG, "an output overlaps an input");
      for (int o2 = o + 1; o2 < 5; ++o2)
        if (overlap(op[o], ob[o], op[o2], ob[o2])) return fail(AS_ERR_INVALID_ARG, "outputs overlap each other");
    }
  }
  as::PlanArgs g;
  memset(&g, 0, sizeof(g));
  g.anchor_norms = anchor_norms; g.local_drift = local_drift; g.weights = weights; g.eps = eps;
  g.alpha = alpha; g.delta = delta; g.ase = ase; g.compute = compute; g.anchor = anchor;
  g.P = P; g.local = local; g.eps_local = eps_local;
  g.group = group > P ? P : group;   // a group of more than P partitions is one group of P
  return hip_status(as::launch_planner_decide(g, stream), "planner_decide launch");
}

as_status as_planner_epsilon(const float* corr_norms, const float* weights, int32_t P, int32_t local,
                             int32_t group, float reuse_fraction, float* eps, hipStream_t stream) {
  const as_status st = check_groups(P, local, group);
  if (st != AS_OK) return st;
  if (!(reuse_fraction >= 0.f && reuse_fraction <= 1.f))
    return fail(AS_ERR_INVALID_ARG, "reuse_fraction=%g outside [0, 1]", (double)reuse_fraction);
  if (!corr_norms || !weights || !eps) return fail(AS_ERR_INVALID_ARG, "corr_norms, weights and eps must not be NULL");
  if (!aligned(corr_norms, 4) || !aligned(weights, 4) || !aligned(eps, 4))
    return fail(AS_ERR_INVALID_ARG, "misaligned pointer");
  if (overlap(eps, 4, corr_norms, (size_t)P * 4) || overlap(eps, 4, weights, (size_t)P * 4))
    return fail(AS_ERR_INVALID_ARG, "eps overlaps an input");
  as::PlanArgs g;
  memset(&g, 0, sizeof(g));
  g.corr_norms = corr_norms; g.weights = weights; g.eps_out = eps;
  g.P = P; g.local = local; g.reuse_fraction = reuse_fraction;
  g.group = group > P ? P : group;
  return hip_status(as::launch_planner_epsilon(g, stream), "planner_epsilon launch");
}
}  // extern "C"
