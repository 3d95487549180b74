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

as_status attn_impl(const void* q, const void* k, const void* v, as_dtype dtype,
                    int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                    const int64_t q_stride[3], const int64_t kv_stride[3],
                    const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                    void* out, float* lse, hipStream_t stream,
                    bool qk_fp8 = false, const float* q_scale = nullptr, const float* k_scale = nullptr) {
  if (dtype != AS_BF16 && dtype != AS_F32) return fail(AS_ERR_INVALID_ARG, "dtype %d is not AS_BF16 or AS_F32", (int)dtype);
  if (state_dtype != AS_BF16 && state_dtype != AS_F32)
    return fail(AS_ERR_INVALID_ARG, "state_dtype %d is not AS_BF16 or AS_F32", (int)state_dtype);
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
  const int64_t rows = B * H * Sq;
  if (rows == 0 || P == 0) return ok();
  if (!q || !k || !v || !out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!q_stride || !kv_stride) return fail(AS_ERR_INVALID_ARG, "NULL stride array");
  if (qk_fp8 && (!q_scale || !k_scale)) return fail(AS_ERR_INVALID_ARG, "q_scale and k_scale must not be NULL");
  if (qk_fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4)))
    return fail(AS_ERR_INVALID_ARG, "q_scale and k_scale must be 4-byte aligned");
  const int64_t esz = dtype == AS_BF16 ? 2 : 4;   // bytes per v element (the widest input)
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
  if (B * H > 65535) return fail(AS_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)(B * H));
  if (Sq > 0x7fffffff || Skv > 0x7fffffff) return fail(AS_ERR_UNSUPPORTED, "sequence length exceeds 2^31-1");
  for (int32_t i = 0; i < P; ++i) {
    const int64_t n = (int64_t)kv_ranges[2 * i + 1] - kv_ranges[2 * i];
    if (n * kv_stride[2] * esz >= ((int64_t)1 << 31)) return fail(AS_ERR_UNSUPPORTED, "kv range %d spans 2^31 bytes or more", i);
  }

  as::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v;
  a.q_sb = q_stride[0]; a.q_sh = q_stride[1]; a.q_ss = q_stride[2];
  a.k_sb = kv_stride[0]; a.k_sh = kv_stride[1]; a.k_ss = kv_stride[2];
  a.out = out; a.lse = lse;
  a.out_bf16 = state_dtype == AS_BF16 ? 1 : 0;
  a.qk_fp8 = qk_fp8 ? 1 : 0;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.B = (int32_t)B; a.H = (int32_t)H; a.Sq = (int32_t)Sq; a.Skv = (int32_t)Skv; a.D = (int32_t)D; a.P = P;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  for (int32_t i = 0; i < 2 * P; ++i) a.ranges[i] = kv_ranges[i];

  if (dtype == AS_BF16) {
    const int bq = as::attn_bf16_rows_per_block((int)D);
    a.n_qtiles = (int32_t)((Sq + bq - 1) / bq);
    if ((int64_t)a.n_qtiles * B * H * P > 0x7fffffff) return fail(AS_ERR_UNSUPPORTED, "grid too large");
    return hip_status(as::launch_attn_bf16(a, stream), "partition_attn bf16 launch");
  }
  const int bq = as::attn_f32_rows_per_block((int)D);
  a.n_qtiles = (int32_t)((Sq + bq - 1) / bq);
  if (B * H * P > 65535) return fail(AS_ERR_UNSUPPORTED, "f32 path: B*H*P=%lld exceeds 65535", (long long)(B * H * P));
  return hip_status(as::launch_attn_f32(a, stream), "partition_attn f32 launch");
}

bool is_state_dtype(as_dtype t) { return t == AS_F32 || t == AS_BF16; }

as_status merge_impl(int32_t n, const void* const* outs, const float* const* lses, as_dtype in_dtype,
                     int64_t rows, int64_t D, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  if (!is_state_dtype(in_dtype) || !is_state_dtype(out_dtype))
    return fail(AS_ERR_INVALID_ARG, "state dtypes must be AS_F32 or AS_BF16");
  if (n < 1 || n > AS_MAX_MERGE) return fail(AS_ERR_INVALID_ARG, "n=%d outside [1, %d]", n, AS_MAX_MERGE);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (D < 4 || D > 1024 || D % 4) return fail(AS_ERR_INVALID_ARG, "D=%lld must be a multiple of 4 in [4, 1024]", (long long)D);
  if (!outs || !lses) return fail(AS_ERR_INVALID_ARG, "NULL pointer list");
  if (rows == 0) return ok();
  if (!out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL output pointer");
  // OUT is read and written 4 elements at a time: 16 bytes of fp32, 8 of bf16
  const size_t ain = in_dtype == AS_BF16 ? 8 : 16, aout = out_dtype == AS_BF16 ? 8 : 16;
  if (!aligned(out, aout) || !aligned(lse, 4))
    return fail(AS_ERR_INVALID_ARG, "out must be %zu-byte and lse 4-byte aligned", aout);
  as::MergeArgs a;
  memset(&a, 0, sizeof(a));
  for (int32_t i = 0; i < n; ++i) {
    if (!outs[i] || !lses[i]) return fail(AS_ERR_INVALID_ARG, "input %d has a NULL pointer", i);
    if (!aligned(outs[i], ain) || !aligned(lses[i], 4)) return fail(AS_ERR_INVALID_ARG, "input %d is misaligned", i);
    if (outs[i] == out || lses[i] == lse) return fail(AS_ERR_INVALID_ARG, "input %d aliases the output", i);
    a.outs[i] = outs[i];
    a.lses[i] = lses[i];
  }
  a.out = out; a.lse = lse; a.rows = rows; a.n = n; a.D = (int32_t)D;
  a.in_bf16 = in_dtype == AS_BF16; a.out_bf16 = out_dtype == AS_BF16;
  a.vec2 = D % 8 == 0 && aligned(out, 16);
  for (int32_t i = 0; i < n; ++i) a.vec2 = a.vec2 && aligned(outs[i], 16);
  return hip_status(as::launch_merge(a, stream), "merge launch");
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
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

as_status as_merge_states(int32_t n, const void* const* outs, const float* const* lses, as_dtype in_dtype,
                          int64_t rows, int64_t D, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  return merge_impl(n, outs, lses, in_dtype, rows, D, out_dtype, out, lse, stream);
}

as_status as_compose_groups(const void* outs, const float* lses, as_dtype in_dtype, int32_t P, int64_t rows,
                            int64_t D, int32_t group, as_dtype out_dtype, void* out, float* lse, hipStream_t stream) {
  if (!is_state_dtype(in_dtype) || !is_state_dtype(out_dtype))
    return fail(AS_ERR_INVALID_ARG, "state dtypes must be AS_F32 or AS_BF16");
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (group < 1 || group > AS_MAX_MERGE) return fail(AS_ERR_INVALID_ARG, "group=%d outside [1, %d]", group, AS_MAX_MERGE);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (D < 4 || D > 1024 || D % 4) return fail(AS_ERR_INVALID_ARG, "D=%lld must be a multiple of 4 in [4, 1024]", (long long)D);
  if (rows == 0) return ok();
  if (!outs || !lses || !out || !lse) return fail(AS_ERR_INVALID_ARG, "NULL pointer");
  if (!aligned(outs, 16) || !aligned(out, 16) || !aligned(lses, 4) || !aligned(lse, 4))
    return fail(AS_ERR_INVALID_ARG, "OUT blocks must be 16-byte and LSE blocks 4-byte aligned");
  const int64_t G = (P + group - 1) / group;
  const size_t ein = in_dtype == AS_BF16 ? 2 : 4, eout = out_dtype == AS_BF16 ? 2 : 4;
  if (overlap(outs, (size_t)(P * rows * D) * ein, out, (size_t)(G * rows * D) * eout) ||
      overlap(lses, (size_t)(P * rows) * 4, lse, (size_t)(G * rows) * 4) ||
      overlap(outs, (size_t)(P * rows * D) * ein, lse, (size_t)(G * rows) * 4) ||
      overlap(lses, (size_t)(P * rows) * 4, out, (size_t)(G * rows * D) * eout))
    return fail(AS_ERR_INVALID_ARG, "outputs overlap the input blocks");
  as::MergeArgs a;
  memset(&a, 0, sizeof(a));
  a.base_out = outs; a.base_lse = lses; a.out = out; a.lse = lse;
  a.rows = rows; a.n = P; a.D = (int32_t)D; a.group = group;
  a.in_bf16 = in_dtype == AS_BF16; a.out_bf16 = out_dtype == AS_BF16;
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

size_t as_partition_contribution_workspace_size(int32_t P, int64_t rows, int64_t rows_per_group) {
  if (P < 1 || P > AS_MAX_PARTITIONS || rows < 0 || rows_per_group < 1 || rows % rows_per_group) return 0;
  const int64_t G = rows / rows_per_group;
  const int64_t chunks = (rows_per_group + as::kContribChunk - 1) / as::kContribChunk;
  return (size_t)(G * chunks * P) * sizeof(float);
}

as_status as_partition_contribution(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group,
                                    float* weights, float* scores, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (P < 1 || P > AS_MAX_PARTITIONS) return fail(AS_ERR_INVALID_ARG, "P=%d outside [1, %d]", P, AS_MAX_PARTITIONS);
  if (rows < 0) return fail(AS_ERR_INVALID_ARG, "rows=%lld is negative", (long long)rows);
  if (rows_per_group < 1) return fail(AS_ERR_INVALID_ARG, "rows_per_group=%lld must be >= 1", (long long)rows_per_group);
  if (rows % rows_per_group) return fail(AS_ERR_INVALID_ARG, "rows=%lld is not a multiple of rows_per_group=%lld",
                                         (long long)rows, (long long)rows_per_group);
  if (rows == 0 || (!weights && !scores)) return ok();
  if (!lse) return fail(AS_ERR_INVALID_ARG, "lse is NULL");
  if (!aligned(lse, 4) || (weights && !aligned(weights, 4)) || (scores && !aligned(scores, 4)))
    return fail(AS_ERR_INVALID_ARG, "misaligned pointer");
  if ((int64_t)P * rows > ((int64_t)1 << 40)) return fail(AS_ERR_UNSUPPORTED, "P*rows too large");
  const size_t need = as_partition_contribution_workspace_size(P, rows, rows_per_group);
  if (scores) {
    if (!workspace) return fail(AS_ERR_INVALID_ARG, "workspace is NULL but scores were requested");
    if (workspace_bytes < need)
      return fail(AS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(AS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  as::ContribArgs a;
  memset(&a, 0, sizeof(a));
  a.lse = lse; a.weights = weights; a.scores = scores;
  a.partial = scores ? static_cast<float*>(workspace) : nullptr;
  a.rows = rows; a.rows_per_group = rows_per_group; a.P = P;
  a.chunks_per_group = (int32_t)((rows_per_group + as::kContribChunk - 1) / as::kContribChunk);
  return hip_status(as::launch_contribution(a, stream), "partition_contribution launch");
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
  as::PlanArgs g;
  memset(&g, 0, sizeof(g));
  g.corr_norms = corr_norms; g.weights = weights; g.eps_out = eps;
  g.P = P; g.local = local; g.reuse_fraction = reuse_fraction;
  g.group = group > P ? P : group;
  return hip_status(as::launch_planner_epsilon(g, stream), "planner_epsilon launch");
}
}  // extern "C"
