// Internal launch interface between the C ABI layer (api.hip) and the kernels.
// Not installed; the public interface is include/as_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "as_attn.h"

namespace as {

// Storage of a state's OUT (the attention kernel's out_kind, the merge kernels' types).
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutFP8 = 2;

// An fp8 state payload of `rows` rows of D: the E4M3 codes [rows][D], then one float32
// factor per row at byte offset rows * D; a value is code * factor of its row. Payloads
// of a block follow each other every payload_bytes (16-byte multiples).
inline int64_t fp8_payload_bytes(int64_t rows, int64_t D) { return rows * D + (rows * 4 + 15) / 16 * 16; }

// Arguments of one partition-attention launch, passed by value as the kernel
// argument (the key ranges travel in the kernarg segment).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh, q_ss;  // element strides of q over (b, h, s)
  int64_t k_sb, k_sh, k_ss;  // element strides of k and v over (b, h, s)
  void* out;                 // [P][B][H][Sq][D] of out_kind (kOutFP8: P payloads)
  float* lse;                // [P][B][H][Sq]
  int32_t B, H, Sq, Skv, D, P;
  int32_t n_qtiles;          // ceil(Sq / rows per workgroup)
  float scale;               // softmax scale
  float scale_log2;          // scale * log2(e)
  int32_t out_kind;          // OUT storage: kOutF32, kOutBF16 (rounded to nearest even) or
                             // kOutFP8 (E4M3 codes with one factor per row: a state payload)
  int32_t qk_fp8;            // q and k are fp8 e4m3, dequantised by q_scale, k_scale
  int32_t v_fp8;             // v is fp8 e4m3 too, dequantised by v_scale (with qk_fp8 only)
  const float* q_scale;      // [B*H] (qk_fp8 only)
  const float* k_scale;      // [B*H] (qk_fp8 only)
  const float* v_scale;      // [B*H] (v_fp8 only)
  int64_t state_rows;        // B*H*Sq: rows of one partition's state
  int64_t payload_bytes;     // kOutFP8: bytes of one partition's state payload
  int32_t split_kr;          // single-partition launches with partial query tiles: of the
                             // C compute units of an XCD, split_kr run only partial tiles
                             // and the others only full ones (0: full tiles first, then
                             // partial ones); split_c = C. Set by the launch.
  int32_t split_c;
  int32_t ranges[2 * AS_MAX_PARTITIONS];
  // Grouped launches (as_partition_attn_grouped): `ranges` holds the non-empty
  // partitions only, packed in group order (P of them); group g holds packed partitions
  // group_starts[g] .. group_starts[g + 1] - 1 and packed partition k is the caller's
  // partition part_index[k]; out/lse are [G][B][H][Sq](D).
  int32_t G;
  const float* fold_out;     // [B][H][Sq][D], composed into group 0's state, or null
  const float* fold_lse;     // [B][H][Sq]
  float* part_lse;           // [caller's P][B][H][Sq] LSE of every partition, or null
  uint16_t group_starts[AS_MAX_PARTITIONS + 1];
  uint16_t part_index[AS_MAX_PARTITIONS];
};

// Sets n floats at p to -inf (the LSE of empty partitions in grouped launches).
hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t stream);

// k-way composition. Pointer mode (group == 0): inputs outs[k], lses[k], k < n.
// Batched mode (group > 0, group-wise composition): n = P slices of one
// partition-major block (base_out [P][rows][D], base_lse [P][rows]); grid.y = group
// index k, whose inputs are slices k*group .. min((k+1)*group, P) - 1; outputs are
// [G][rows][D] and [G][rows].
struct MergeArgs {
  const void* outs[AS_MAX_MERGE];   // [rows][D] of in_kind each (kOutFP8: a payload)
  const float* lses[AS_MAX_MERGE];
  const void* base_out;
  const float* base_lse;
  void* out;                        // [rows][D] of out_kind (kOutFP8: a payload)
  float* lse;
  int64_t rows;
  int32_t n;
  int32_t D;
  int32_t group;
  int32_t in_kind, out_kind;        // kOutF32, kOutBF16 or kOutFP8
  int64_t payload_bytes;            // fp8 payload of `rows` rows (fp8_payload_bytes)
  int32_t vec2;   // bf16 inputs: every OUT pointer 16-byte aligned and D % 8 == 0 (16-byte lane loads)
};

struct ContribArgs {
  const float* lse;   // [P][rows]
  float* weights;     // [P][rows] or null
  float* scores;      // [G][P] or null
  float* partial;     // [G][chunks_per_group][P] workspace or null
  int64_t rows;
  int64_t rows_per_group;
  int32_t P;
  int32_t chunks_per_group;
};

// Rows of the query shard handled by one workgroup of the bf16 kernel.
int attn_bf16_rows_per_block(int D);
int attn_f32_rows_per_block(int D);

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t stream);   // bf16 or fp8 q/k (qk_fp8)
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t stream);    // fp8 q/k
hipError_t launch_attn_fp8v(const AttnArgs& a, hipStream_t stream);   // fp8 q/k/v
hipError_t launch_attn_grouped_fp8v(const AttnArgs& a, hipStream_t stream);   // grouped, fp8 q/k/v
hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// State norms: slice i of n floats is split into chunks of norms_chunk(P, n)
// elements (a multiple of 1024, so every thread of a 256-thread workgroup reads
// whole 16-byte vectors); one fp64 partial per (slice, chunk) goes to the workspace.
struct NormArgs {
  const float* a;      // [P][n]
  const float* b;      // [P][n] or null
  float* norms;        // [P]
  double* partial;     // [P][chunks]
  int64_t n;
  int64_t chunk;
  int32_t P;
  int32_t chunks;
};

inline int64_t norms_chunk(int32_t P, int64_t n) {
  int64_t c = (n * P + 2047) / 2048;            // about 2048 workgroups in all
  c = (c + 1023) / 1024 * 1024;
  return c < 4096 ? 4096 : (c > 262144 ? 262144 : c);
}
inline int64_t norms_chunks(int32_t P, int64_t n) {
  const int64_t c = norms_chunk(P, n);
  return n == 0 ? 1 : (n + c - 1) / c;
}

struct PlanArgs {
  const float* anchor_norms;   // decide: [P]
  const float* local_drift;    // decide: [1]
  const float* corr_norms;     // epsilon: [P]
  const float* weights;        // [P]
  const float* eps;            // decide: [1]
  float* alpha;                // decide: [P] or null
  float* delta;                // decide: [P] or null
  float* ase;                  // decide: [G] or null
  int32_t* compute;            // decide: [G]
  int32_t* anchor;             // decide: [1]
  float* eps_out;              // epsilon: [1]
  int32_t P, local, group;
  float eps_local;
  float reuse_fraction;
};

hipError_t launch_state_norms(const NormArgs& a, hipStream_t stream);
hipError_t launch_planner_decide(const PlanArgs& a, hipStream_t stream);
hipError_t launch_planner_epsilon(const PlanArgs& a, hipStream_t stream);

// Contribution: rows are processed in chunks of this many rows per workgroup.
constexpr int kContribChunk = 256;
hipError_t launch_contribution(const ContribArgs& a, hipStream_t stream);

// Library-owned scratch of the allocation-free contribution entry point: its size,
// and its device address on the current device (looked up once per device).
constexpr size_t kContribScratchBytes = AS_CONTRIBUTION_SCRATCH_BYTES;
hipError_t contribution_scratch(float** ptr);

}  // namespace as
