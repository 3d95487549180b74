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
 *   - Aliasing: outputs must not overlap inputs or one another. Every call checks
 *     the byte ranges its arguments span (for strided tensors, first to last
 *     element) and returns AS_ERR_INVALID_ARG on an overlap.
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
  AS_BF16 = 0,     /* bfloat16 Q/K/V: QK^T and PV on bf16 MFMA, fp32 accumulation and softmax */
  AS_F32 = 1,      /* float32 Q/K/V: fp32 arithmetic throughout (accuracy path) */
  AS_FP8_E4M3 = 2  /* as an input dtype (as_partition_attn_grouped): fp8 E4M3 Q/K codes with
                      per-(b, h) factors (as for as_partition_attn_fp8); as a state dtype: an
                      fp8 state payload (see "Compact states" below) */
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
 * scale      softmax scale (callers pass 1/sqrt(D) for standard attention); finite and
 *            >= 0. scale = 0 weighs every key of a range equally: OUT_i = mean of V over
 *            the range, LSE_i = log(n_i).
 * out        DEVICE float32 [P][B][H][Sq][D], contiguous, 16-byte aligned.
 * lse        DEVICE float32 [P][B][H][Sq], contiguous, 4-byte aligned.
 *            out and lse must not overlap each other or q, k, v (checked).
 * Alignment: q, k, v 16-byte aligned; strides multiples of 8 elements (bf16) or
 * 4 elements (f32); stride_s >= D. B*H <= 65535; max(n_i, 128) * kv_stride[2] *
 * element size < 2^31 bytes for every range (else AS_ERR_UNSUPPORTED).
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
 * out, lse   DEVICE float32 [rows][D] (16-byte aligned) and [rows]; must not overlap any
 *            input or each other (byte ranges checked).
 * If rows == 0 nothing is enqueued.
 */
as_status as_merge(int32_t n, const float* const* outs, const float* const* lses,
                   int64_t rows, int64_t D, float* out, float* lse, hipStream_t stream);

/*
 * Compact states and group-wise composition.
 *   Source: DiTango review page (pith.science), "If this is right": an attention
 *   state is about half the size of the KV it summarises, and composed states can
 *   be merged into coarser groups under memory pressure; the free-parameter ledger
 *   gives the group size g (4, 8 or 16 explored).
 * A state's OUT may be stored as float32 (AS_F32), bfloat16 (AS_BF16, rounded to
 * nearest even) or as an fp8 state payload (AS_FP8_E4M3); LSE is always float32. A bf16
 * state of D = 128 takes 2D + 4 = 260 bytes per query row against 516 for fp32; an fp8
 * one D + 8 = 136. All arithmetic is fp32 whatever the storage.
 *
 * fp8 state payload (sources: the FastUSP page (mlsanity), abstract: attention traffic
 * quantised to FP8; its prior work, "FP8 Formats for Deep Learning", defines E4M3): the
 * OUT of a state of `rows` rows of D is one byte block of as_state_bytes(AS_FP8_E4M3,
 * rows, D) = rows*D + 16*ceil(4*rows/16) bytes:
 *   codes    uint8 [rows][D] at byte 0: OCP E4M3 ("e4m3fn") codes, row-major;
 *   factors  float32 [rows] at byte rows*D (16-byte aligned when D % 16 == 0);
 * element (r, d) stands for decode(codes[r][d]) * factors[r]. Writers set
 * factors[r] = amax_r / 448 with amax_r = max_d |OUT[r][d]| (the fp32 value before
 * storage) and codes[r][d] = E4M3 of OUT[r][d] * (448 / amax_r) rounded to nearest even
 * (clamped to +-448), both quotients rounded float32; a zero row (an empty state included)
 * has codes 0 and factor 0. A block of n fp8 states (P partitions, G groups) is n payloads
 * back to back, payload i at byte i * as_state_bytes(AS_FP8_E4M3, rows, D). fp8 states
 * need D in {32, 64, 128, 256} (attention: 64 or 128).
 */

/*
 * as_state_bytes - bytes of one state's OUT storage: rows*D*4 (AS_F32), rows*D*2
 * (AS_BF16) or the fp8 payload size above (AS_FP8_E4M3). Returns 0 for an invalid
 * dtype or sizes (rows < 0, D outside [1, 1024]).
 */
size_t as_state_bytes(as_dtype state_dtype, int64_t rows, int64_t D);

/*
 * as_partition_attn_states - as_partition_attn with the OUT storage type chosen
 * by state_dtype (AS_F32 gives exactly as_partition_attn). out is DEVICE
 * [P][B][H][Sq][D] of state_dtype, contiguous, 16-byte aligned; for AS_FP8_E4M3 it is a
 * block of P fp8 payloads of rows = B*H*Sq (row index (b*H + h)*Sq + s), whose codes
 * and factors are those of the fp32 OUT the call computes. AS_FP8_E4M3 states need
 * dtype AS_BF16 (else AS_ERR_UNSUPPORTED). Every other argument and rule is as for
 * as_partition_attn.
 */
as_status as_partition_attn_states(const void* q, const void* k, const void* v, as_dtype dtype,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                   const int64_t q_stride[3], const int64_t kv_stride[3],
                                   const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                   void* out, float* lse, hipStream_t stream);

/*
 * as_partition_attn_fp8 - as_partition_attn_states with 8-bit floating-point
 * queries and keys.
 *   Sources: the DiTango review page (pith.science) cites SageAttention, 8-bit
 *   attention for plug-and-play inference, among its references; the FastUSP page
 *   (mlsanity) quantises attention traffic to FP8 and builds on "FP8 Formats for
 *   Deep Learning", which defines the E4M3 format used here.
 * q and k hold FP8 E4M3 codes, one byte per element, in the OCP "e4m3fn" encoding
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; largest
 * finite value 448; torch.float8_e4m3fn). v is bfloat16. A code c of batch b and
 * head h stands for the value c * q_scale[b*H + h] in q and c * k_scale[b*H + h] in
 * k, so the states are those of as_partition_attn on the dequantised Q and K and
 * the given V:  z_j = scale * < q_scale[bh] * Q8_r , k_scale[bh] * K8_j >.
 * S = K Q^T runs on the fp8 MFMA (exact products, fp32 accumulation); softmax, P and
 * PV are as in the bf16 path.
 *
 * q_scale, k_scale  DEVICE float32 [B*H], 4-byte aligned; values must be finite (not
 *                   checked: they are device memory). Any sign is allowed: a zero
 *                   factor weighs the keys equally, as scale = 0 does.
 * q_stride          element (= byte) strides of q over (b, h, s).
 * kv_stride         element strides of k and v over (b, h, s): k's row stride is
 *                   kv_stride[2] bytes, v's 2 * kv_stride[2] bytes. All strides are
 *                   multiples of 16 elements.
 * D                 64 or 128 (else AS_ERR_UNSUPPORTED).
 * Every other argument and rule is as for as_partition_attn_states.
 */
as_status as_partition_attn_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                const float* k_scale, int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t D,
                                const int64_t q_stride[3], const int64_t kv_stride[3],
                                const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                void* out, float* lse, hipStream_t stream);

/*
 * as_partition_attn_fp8_qkv - as_partition_attn_fp8 with fp8 values too: q, k and v all
 * hold E4M3 codes, and a code of v of batch b and head h stands for code * v_scale[b*H + h].
 *   Source: the FastUSP page (mlsanity), abstract: the attention traffic, keys and
 *   values included, quantised to FP8.
 * The states are those of as_partition_attn on the dequantised Q, K and V. The value codes
 * are widened to bfloat16 (exactly) for PV; v_scale multiplies OUT at the end.
 * v_scale    DEVICE float32 [B*H], 4-byte aligned, finite, any sign (not checked: device
 *            memory).
 * kv_stride  element (= byte) strides of k and v over (b, h, s), multiples of 16.
 * Every other argument and rule is as for as_partition_attn_fp8 (state_dtype AS_F32,
 * AS_BF16 or AS_FP8_E4M3).
 */
as_status as_partition_attn_fp8_qkv(const void* q, const void* k, const void* v, const float* q_scale,
                                    const float* k_scale, const float* v_scale, int64_t B, int64_t H, int64_t Sq,
                                    int64_t Skv, int64_t D, const int64_t q_stride[3], const int64_t kv_stride[3],
                                    const int32_t* kv_ranges, int32_t P, float scale, as_dtype state_dtype,
                                    void* out, float* lse, hipStream_t stream);

/*
 * as_partition_attn_grouped - partition attention whose epilogue composes the states of
 * consecutive partitions. For every group g of the range list (partitions
 * group_starts[g] .. group_starts[g + 1] - 1) it writes the composed state of the group's
 * partitions, i.e. as_merge of their as_partition_attn states, from one pass over their
 * keys without writing any per-partition OUT; optionally the LSE of every partition; and
 * optionally composes a given state (such as the cached composed state of other
 * partitions) into group 0's result.
 *   Source: DiTango review page (pith.science), referee report summary ("ring-based
 *   attention composition" and "memory-aware state merging"); axiom ledger (Eq. 1-2:
 *   associative, commutative composition); "If this is right" (composed states merged
 *   into coarser groups).
 *
 * dtype         AS_BF16 (q, k, v bfloat16) or AS_FP8_E4M3 (q, k E4M3 codes with q_scale,
 *               k_scale and strides as for as_partition_attn_fp8; v bfloat16, or E4M3
 *               codes when v_scale is given, as for as_partition_attn_fp8_qkv). D is 64
 *               or 128.
 * q_scale, k_scale, v_scale  as for as_partition_attn_fp8 and as_partition_attn_fp8_qkv
 *               (AS_FP8_E4M3 only; ignored for AS_BF16); v_scale NULL: v is bfloat16.
 * kv_ranges, P  as for as_partition_attn, with 1 <= P <= AS_MAX_PARTITIONS.
 * group_starts  HOST int32 [G + 1] with 0 = group_starts[0] <= ... <= group_starts[G] = P;
 *               1 <= G <= AS_MAX_PARTITIONS; an empty group gives (0, -inf). Groups are
 *               scheduled in list order: listing long groups first starts them first.
 * fold_out, fold_lse  DEVICE float32 [B][H][Sq][D] (16-byte aligned) and [B][H][Sq], or
 *               both NULL: a state composed into group 0's result as as_merge would.
 * out, lse      DEVICE float32 [G][B][H][Sq][D] (16-byte aligned) and [G][B][H][Sq].
 * part_lse      DEVICE float32 [P][B][H][Sq] or NULL: the LSE of every partition, equal to
 *               as_partition_attn's lse (e.g. for as_partition_contribution) up to rounding,
 *               with one exception: a partition's sum is taken against the running max of
 *               its group, so a partition whose every score lies more than 87 below the
 *               largest score of the earlier keys of its group (weight under e^-87 of
 *               theirs, below fp32's normal range either way) may come out smaller, down
 *               to -inf.
 * Outputs must not overlap each other or any input (checked). All other arguments and
 * rules are as for as_partition_attn.
 */
as_status as_partition_attn_grouped(const void* q, const void* k, const void* v, as_dtype dtype,
                                    const float* q_scale, const float* k_scale, const float* v_scale,
                                    int64_t B, int64_t H,
                                    int64_t Sq, int64_t Skv, int64_t D, const int64_t q_stride[3],
                                    const int64_t kv_stride[3], const int32_t* kv_ranges, int32_t P,
                                    const int32_t* group_starts, int32_t G, float scale, const float* fold_out,
                                    const float* fold_lse, float* out, float* lse, float* part_lse,
                                    hipStream_t stream);

/*
 * as_merge_states - as_merge for states whose OUT is stored as in_dtype, writing an
 * OUT of out_dtype (AS_F32/AS_F32 gives exactly as_merge). outs: HOST array of n
 * DEVICE pointers, each [rows][D] of in_dtype (AS_FP8_E4M3: a payload of rows rows);
 * out: DEVICE [rows][D] of out_dtype (or a payload). OUT pointers are 16-byte aligned
 * for fp32 and fp8 payloads and 8-byte aligned for bf16 (a slice of a bf16 block with D
 * a multiple of 4 always is). An fp8 input is read as decode(code) * factor of its row;
 * an fp8 output is written by the payload rule from the fp32 result. With an fp8 state
 * D must be 32, 64, 128 or 256 (else AS_ERR_UNSUPPORTED). Other rules as for as_merge.
 */
as_status as_merge_states(int32_t n, const void* const* outs, const float* const* lses, as_dtype in_dtype,
                          int64_t rows, int64_t D, as_dtype out_dtype, void* out, float* lse, hipStream_t stream);

/*
 * as_compose_groups - group-wise composition: the states of partitions
 * k*group .. min((k+1)*group, P) - 1 of a partition-major block are composed (as in
 * as_merge) into one state per group k, for all G = ceil(P / group) groups in one
 * launch.
 *
 * outs, lses  DEVICE [P][rows][D] of in_dtype (16-byte aligned; AS_FP8_E4M3: P payloads)
 *             and float32 [P][rows] (as written by as_partition_attn_states).
 * P           1 <= P <= AS_MAX_PARTITIONS.   group: 1 <= group <= AS_MAX_MERGE.
 * rows, D     rows >= 0; D a multiple of 4, 4 <= D <= 1024.
 * out, lse    DEVICE [G][rows][D] of out_dtype (16-byte aligned; AS_FP8_E4M3: G payloads)
 *             and float32 [G][rows]; must not overlap the input blocks.
 * fp8 states as for as_merge_states.
 */
as_status as_compose_groups(const void* outs, const float* lses, as_dtype in_dtype, int32_t P, int64_t rows,
                            int64_t D, int32_t group, as_dtype out_dtype, void* out, float* lse, hipStream_t stream);

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

/*
 * as_partition_contribution_noalloc - as_partition_contribution for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. It takes no workspace; the per-chunk partial sums of the score
 * reduction live in a static device buffer of AS_CONTRIBUTION_SCRATCH_BYTES that the
 * library holds on every device it runs on until the process ends. Neither this call
 * nor its first-call setup allocates or frees memory.
 *
 * Sizes: with scores requested, as_partition_contribution_workspace_size(P, rows,
 * rows_per_group) must not exceed AS_CONTRIBUTION_SCRATCH_BYTES, else AS_ERR_INVALID_ARG
 * (the long-video anchor, 32 partitions x 24 groups of 3840 rows, needs 46080 bytes).
 * Sharing: every call on one device uses that device's single buffer, and it keeps the
 * last call's contents (nothing in it needs to start at zero: each call overwrites what
 * it reads). Calls whose work overlaps in time on one device (different streams, or
 * threads without ordering between them) race on it; issue them on one stream or order
 * them. The stream must belong to the current device; the first call on a device
 * looks up the buffer's address there. Every other argument and rule is as for
 * as_partition_contribution.
 */
#define AS_CONTRIBUTION_SCRATCH_BYTES ((size_t)1 << 20)
as_status as_partition_contribution_noalloc(const float* lse, int32_t P, int64_t rows, int64_t rows_per_group,
                                            float* weights, float* scores, hipStream_t stream);

/*
 * Anchor-guided planner statistics.
 *   Source: DiTango review page (pith.science): "What carries the argument" (the
 *   group error ASE(G_i, t) = sum over the group of w(j, t) * delta(j, t, t_c), Eq. 12),
 *   the free-parameter ledger (scale ratio alpha(i) = ||AS_ta(i)|| / ||AS_ta(i_loc)||,
 *   Eq. 9; group size g; local threshold eps_local and percentile threshold eps of
 *   Algorithm 1) and the referee report on section 4.1.2 (drift model
 *   delta(i, t, t_a) = alpha(i) * ||AS_t(i_loc) - AS_ta(i_loc)||, Eq. 10, and the
 *   reuse decision of Eq. 13).
 *   ||AS|| is taken as the L2 norm of the OUT part of a state over the whole query
 *   shard (LSE excluded).
 */

/*
 * as_state_norms_workspace_size - bytes of device workspace as_state_norms needs
 * for these sizes (one fp64 partial sum per chunk of each slice). Returns 0 for
 * invalid sizes.
 */
size_t as_state_norms_workspace_size(int32_t P, int64_t n);

/*
 * as_state_norms - L2 norms of P state slices or of their differences:
 *   norms[i] = sqrt(sum_e (a[i][e] - b[i][e])^2),   or sqrt(sum_e a[i][e]^2) if b is NULL.
 * Differences and squares are formed and summed in fp64 in a fixed order, so the
 * result (rounded to fp32) is bitwise reproducible.
 *
 * a, b       DEVICE float32 [P][n], contiguous (slice i starts at element i*n),
 *            16-byte aligned; b may be NULL. For a1's output, a slice is one
 *            partition's OUT: n = B*H*Sq*D.
 * P          1 <= P <= AS_MAX_PARTITIONS.
 * n          >= 0 and a multiple of 4. n == 0 gives norms of 0.
 * norms      DEVICE float32 [P], 4-byte aligned.
 * workspace  DEVICE buffer of at least as_state_norms_workspace_size(P, n) bytes,
 *            16-byte aligned; its contents on entry do not matter.
 */
as_status as_state_norms(const float* a, const float* b, int32_t P, int64_t n, float* norms,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * as_planner_decide - one planning step. Partitions form contiguous groups of
 * `group`: group k holds partitions k*group .. min((k+1)*group, P) - 1 (the last
 * group may be shorter); the local group is local / group. With d = local_drift[0]:
 *   alpha[i]   = anchor_norms[i] / anchor_norms[local]                  (Eq. 9)
 *   delta[i]   = alpha[i] * d                                           (Eq. 10)
 *   ase[k]     = sum over j in group k of weights[j] * delta[j]         (Eq. 12)
 *   compute[k] = 1 if k is the local group or ase[k] > eps[0], else 0   (Eq. 13: 0 = reuse)
 *   anchor[0]  = 1 if d > eps_local, else 0     (Algorithm 1: a new anchor step is due)
 * fp32 arithmetic; group sums in ascending partition order.
 *
 * anchor_norms  DEVICE float32 [P]: ||OUT_ta(i)|| (as_state_norms on the anchor step's
 *               states); anchor_norms[local] must be > 0.
 * local_drift   DEVICE float32 [1]: ||OUT_t(local) - OUT_ta(local)|| (as_state_norms, P = 1).
 * weights       DEVICE float32 [P]: w(i) of the anchor step (as_partition_contribution
 *               scores with one group of all rows).
 * eps           DEVICE float32 [1]: the reuse threshold (as_planner_epsilon or the caller's).
 * P, local      1 <= P <= AS_MAX_PARTITIONS, 0 <= local < P.   group >= 1.
 * eps_local     finite.
 * alpha, delta  DEVICE float32 [P] or NULL (not written).   ase: DEVICE float32 [G] or NULL.
 * compute       DEVICE int32 [G], G = ceil(P / group).   anchor: DEVICE int32 [1].
 */
as_status as_planner_decide(const float* anchor_norms, const float* local_drift, const float* weights,
                            const float* eps, int32_t P, int32_t local, int32_t group, float eps_local,
                            float* alpha, float* delta, float* ase, int32_t* compute, int32_t* anchor,
                            hipStream_t stream);

/*
 * as_planner_epsilon - the reuse threshold of Algorithm 1 from anchor correction errors.
 *   E[k]   = sum over j in group k of weights[j] * corr_norms[j]   (groups as above)
 *   m      = floor(float(reuse_fraction) * float(G')) over the G' = G - 1 non-local
 *            groups (float32 product)
 *   eps[0] = the m-th smallest E[k] over the non-local groups (ties broken by group
 *            index), or -inf when m == 0 (nothing is reused).
 * With this eps, m non-local groups have E[k] <= eps.
 *
 * corr_norms      DEVICE float32 [P]: ||OUT_ta(j) - OUT_tc(j)|| between the anchor step's
 *                 fresh states and the states cached before it (as_state_norms).
 * weights         DEVICE float32 [P] (as in as_planner_decide).
 * reuse_fraction  target fraction of the non-local groups to reuse, 0 <= R <= 1.
 * eps             DEVICE float32 [1].
 */
as_status as_planner_epsilon(const float* corr_norms, const float* weights, int32_t P, int32_t local,
                             int32_t group, float reuse_fraction, float* eps, hipStream_t stream);

/* Static description of a status code. */
const char* as_status_string(as_status s);

/* Detail of the last failure on the calling thread ("" if none). Valid until the next call. */
const char* as_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AS_ATTN_H */
