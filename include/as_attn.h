/*
 * as_attn.h - C ABI for partition-wise attention states on AMD Instinct MI355X (gfx950).
 *
 * An attention state of query rows against one KV partition i is the pair
 * AS(i) = (OUT(i), LSE(i)): the attention output restricted to the keys of
 * partition i (normalised within the partition) and the log-sum-exp of the
 * scaled scores over those keys. States of disjoint partitions compose
 * associatively and commutatively into the state of their union; a state
 * composed of every partition is exact full attention.
 *   Source: "DiTango: Cost-Effective Parallel Diffusion Generation with Selective
 *   Attention State Reuse" (pith.science review page), sections "What carries the
 *   argument" and the axiom ledger (Eq. 1-2); the free-parameter ledger and the
 *   Fig. 8 caption (Eq. 8) for the partition importance weight.
 *
 * Conventions for every call:
 *   - Ownership: the caller owns all device buffers. The library never allocates,
 *     frees or retains device memory. Host arrays passed in (kv_ranges, pointer
 *     lists) are read during the call only.
 *   - Execution: work is enqueued asynchronously on `stream` (0 = the null stream);
 *     outputs are valid once the stream has reached the enqueued work. No call
 *     synchronises. Calls are reentrant and thread-safe.
 *   - Validation: every argument is checked on the host before any HIP call. An
 *     invalid argument returns AS_ERR_INVALID_ARG, an unsupported but valid
 *     shape returns AS_ERR_UNSUPPORTED; in both cases nothing is enqueued.
 *     A failed launch returns AS_ERR_HIP. as_last_error() gives the detail.
 *     Nothing throws across the ABI.
 *   - Aliasing: outputs must not overlap inputs.
 *   - Floating point: inputs must be finite (NaN/Inf inputs give undefined
 *     results); -inf in an LSE input marks an empty state.
 */
#ifndef AS_ATTN_H
#define AS_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AS_OK = 0,
  AS_ERR_INVALID_ARG = 1,
  AS_ERR_UNSUPPORTED = 2,
  AS_ERR_HIP = 3
} as_status;

typedef enum {
  AS_BF16 = 0, /* bfloat16 Q/K/V: QK^T and PV on bf16 MFMA, fp32 accumulation and softmax */
  AS_F32 = 1   /* float32 Q/K/V: fp32 arithmetic throughout (accuracy path) */
} as_dtype;

#define AS_MAX_PARTITIONS 256 /* partitions per as_partition_attn call */
#define AS_MAX_MERGE 64       /* states per as_merge call */

/*
 * as_partition_attn - attention states of a query shard against P key ranges.
 *
 * Computes, for every batch b, head h, query row r and partition i with key
 * range [s_i, e_i):
 *   z_j   = scale * <Q[b,h,r,:], K[b,h,j,:]>          for j in [s_i, e_i)
 *   LSE_i = log(sum_j exp(z_j))                         (natural log)
 *   OUT_i = sum_j exp(z_j - LSE_i) * V[b,h,j,:]
 * An empty range (s_i == e_i) yields OUT_i = 0 and LSE_i = -inf. No mask.
 * (DiTango review page, "What carries the argument": AS(i) = (OUT(i), LSE(i)).)
 *
 * q          DEVICE [B][H][Sq][D] of `dtype`, element strides q_stride = {b, h, s}, d contiguous.
 * k, v       DEVICE [B][H][Skv][D] of `dtype`, both with element strides kv_stride = {b, h, s}.
 * dtype      AS_BF16: D must be 64 or 128. AS_F32: D a multiple of 4, 4..128.
 * kv_ranges  HOST int32 [P][2] = {s_i, e_i} with 0 <= s_i <= e_i <= Skv. Ranges may
 *            overlap, repeat or be empty. 0 <= P <= AS_MAX_PARTITIONS.
 * scale      softmax scale (callers pass 1/sqrt(D) for standard attention); finite.
 * out        DEVICE float32 [P][B][H][Sq][D], contiguous, 16-byte aligned.
 * lse        DEVICE float32 [P][B][H][Sq], contiguous, 4-byte aligned.
 * Alignment: q, k, v 16-byte aligned; strides multiples of 8 elements (bf16) or
 * 4 elements (f32); stride_s >= D. B*H <= 65535; a range spans < 2^31 bytes.
 * If B*H*Sq == 0 or P == 0 nothing is enqueued and AS_OK is returned.
 */
as_status as_partition_attn(const void* q, const void* k, const void* v, as_dtype dtype,
                            int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                            const int64_t q_stride[3], const int64_t kv_stride[3],
                            const int32_t* kv_ranges, int32_t P, float scale,
                            float* out, float* lse, hipStream_t stream);

/*
 * as_merge - composition of n attention states into one.
 *
 * Per row, with M = max_k LSE_k:
 *   M == -inf (every input empty):  OUT = 0, LSE = -inf
 *   otherwise a_k = exp(LSE_k - M), S = sum_k a_k,
 *             LSE = M + log(S), OUT = sum_k (a_k / S) * OUT_k
 * Composing with an empty state (0, -inf) returns the other state bit for bit.
 * (DiTango review page, axiom ledger, Eq. 1-2: states compose associatively and
 * commutatively; "What carries the argument": cached composed states.)
 *
 * n          1 <= n <= AS_MAX_MERGE.
 * outs       HOST array of n DEVICE pointers, each float32 [rows][D] contiguous, 16-byte aligned.
 * lses       HOST array of n DEVICE pointers, each float32 [rows].
 * rows, D    rows >= 0; D a multiple of 4, 4 <= D <= 1024.
 * out, lse   DEVICE float32 [rows][D] (16-byte aligned) and [rows]; must not overlap any input.
 * If rows == 0 nothing is enqueued.
 */
as_status as_merge(int32_t n, const float* const* outs, const float* const* lses,
                   int64_t rows, int64_t D, float* out, float* lse, hipStream_t stream);

/*
 * as_partition_contribution_workspace_size - bytes of device workspace that
 * as_partition_contribution needs to compute scores for these sizes (per-chunk
 * partial sums of the group reduction). Returns 0 for invalid sizes.
 */
size_t as_partition_contribution_workspace_size(int32_t P, int64_t rows, int64_t rows_per_group);

/*
 * as_partition_contribution - per-row partition weights and per-group scores.
 *
 * Per row r (DiTango review page, free-parameter ledger and Fig. 8 caption,
 * Eq. 8: the importance of partition i is the softmax of LSE over partitions):
 *   L* = log(sum_i exp(LSE[i][r]))
 *   w[i][r] = exp(LSE[i][r] - L*)     (0 where LSE = -inf; all 0 if every LSE is -inf)
 * scores[g][i] = mean of w[i][r] over the rows_per_group rows of group g
 * (rows g*rows_per_group ... (g+1)*rows_per_group - 1). The reduction order is
 * fixed, so scores are bitwise deterministic run to run.
 *
 * lse        DEVICE float32 [P][rows] (partition-major, as written by as_partition_attn).
 * P          1 <= P <= AS_MAX_PARTITIONS.
 * rows_per_group  >= 1 and divides rows.
 * weights    DEVICE float32 [P][rows] or NULL (not written).
 * scores     DEVICE float32 [rows/rows_per_group][P] or NULL (not computed).
 * workspace  DEVICE buffer of at least as_partition_contribution_workspace_size(...)
 *            bytes, 16-byte aligned; may be NULL when scores is NULL. Its contents
 *            on entry do not matter; it is overwritten.
 */
as_status as_partition_contribution(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group,
                                    float* weights, float* scores, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* as_status_string(as_status s);

/* Detail of the last failure on the calling thread ("" if none). Valid until the next call. */
const char* as_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AS_ATTN_H */
