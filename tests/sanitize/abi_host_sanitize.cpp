// Drives every entry point of the C ABI (include/as_attn.h) on the host, with the kernel
// launchers replaced by recorders (launch_stubs.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer. Covers: argument packing of valid calls (what a launch
// would receive), rejection of invalid ones, host arrays sized exactly to their count
// (so an over-read is reported), and sizes whose products overflow 64 bits.
// Exit status 0 and "abi sanitize ok" on success; a failed check prints and aborts.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <memory>
#include <vector>

#include "as_attn.h"
#include "launch_stubs.h"

#define CHECK(cond)                                                                  \
  do {                                                                               \
    if (!(cond)) {                                                                   \
      fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, __LINE__, \
              #cond, as_last_error());                                               \
      abort();                                                                       \
    }                                                                                \
  } while (0)

namespace {

template <typename T>
void* fake(T addr) { return reinterpret_cast<void*>(static_cast<uintptr_t>(addr)); }

// kv ranges in a heap array of exactly 2 * P entries
std::unique_ptr<int32_t[]> ranges(const std::vector<int32_t>& flat) {
  std::unique_ptr<int32_t[]> r(new int32_t[flat.size() ? flat.size() : 1]);
  for (size_t i = 0; i < flat.size(); ++i) r[i] = flat[i];
  return r;
}

void attn_calls() {
  const int64_t B = 2, H = 3, Sq = 300, Skv = 1000, D = 128;
  const int64_t qs[3] = {H * Sq * D, Sq * D, D}, ks[3] = {H * Skv * D, Skv * D, D};
  const std::vector<int32_t> flat = {0, 200, 200, 201, 201, 201, 201, 777, 777, 1000, 100, 300, 0, 1000};
  auto r = ranges(flat);
  const int32_t P = (int32_t)flat.size() / 2;
  void *q = fake(0x10000000), *k = fake(0x20000000), *v = fake(0x30000000);
  void *out = fake(0x40000000), *lse = fake(0x50000000);
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.088f, (float*)out, (float*)lse,
                          nullptr) == AS_OK);
  CHECK(strcmp(stub::last.kind, "attn_bf16") == 0);
  const as::AttnArgs& a = stub::last.attn;
  CHECK(a.B == B && a.H == H && a.Sq == Sq && a.Skv == Skv && a.D == D && a.P == P && a.n_qtiles == 2);
  CHECK(a.q_ss == D && a.k_sh == Skv * D && a.out == out && a.lse == lse && a.out_kind == 0 && a.qk_fp8 == 0);
  for (int i = 0; i < 2 * P; ++i) CHECK(a.ranges[i] == flat[i]);
  CHECK(fabsf(a.scale_log2 - 0.088f * 1.44269504f) < 1e-6f);

  // compact states, fp8 q/k, f32 path
  CHECK(as_partition_attn_states(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.f, AS_BF16, out,
                                 (float*)lse, nullptr) == AS_OK);
  CHECK(stub::last.attn.out_kind == 1 && stub::last.attn.scale_log2 == 0.f);
  float* qsc = (float*)fake(0x60000000);
  float* ksc = (float*)fake(0x60001000);
  CHECK(as_partition_attn_fp8(q, k, v, qsc, ksc, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.088f, AS_F32, out,
                              (float*)lse, nullptr) == AS_OK);
  CHECK(stub::last.attn.qk_fp8 == 1 && stub::last.attn.q_scale == qsc && stub::last.attn.k_scale == ksc);
  CHECK(stub::last.attn.v_fp8 == 0);
  // fp8 state payloads: P payloads of B*H*Sq rows, factors after the codes
  const int64_t rows = B * H * Sq;
  CHECK(as_state_bytes(AS_FP8_E4M3, rows, D) == (size_t)(rows * D + (4 * rows + 15) / 16 * 16));
  CHECK(as_state_bytes(AS_BF16, rows, D) == (size_t)(rows * D * 2) && as_state_bytes((as_dtype)7, rows, D) == 0);
  CHECK(as_partition_attn_states(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.1f, AS_FP8_E4M3, out,
                                 (float*)lse, nullptr) == AS_OK);
  CHECK(stub::last.attn.out_kind == 2 && stub::last.attn.state_rows == rows &&
        stub::last.attn.payload_bytes == (int64_t)as_state_bytes(AS_FP8_E4M3, rows, D));
  // fp8 q/k/v: v's factors; an output over them is refused; f32 inputs cannot write fp8 states
  float* vsc = (float*)fake(0x60002000);
  CHECK(as_partition_attn_fp8_qkv(q, k, v, qsc, ksc, vsc, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.088f,
                                  AS_FP8_E4M3, out, (float*)lse, nullptr) == AS_OK);
  CHECK(stub::last.attn.v_fp8 == 1 && stub::last.attn.v_scale == vsc && stub::last.attn.out_kind == 2);
  CHECK(as_partition_attn_fp8_qkv(q, k, v, qsc, ksc, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.088f, AS_F32,
                                  out, (float*)lse, nullptr) == AS_ERR_INVALID_ARG);
  CHECK(as_partition_attn_fp8_qkv(q, k, v, qsc, ksc, vsc, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.088f, AS_F32,
                                  vsc - 4, (float*)lse, nullptr) == AS_ERR_INVALID_ARG);
  const int64_t qs40[3] = {H * Sq * 40, Sq * 40, 40}, ks40[3] = {H * Skv * 40, Skv * 40, 40};
  CHECK(as_partition_attn(q, k, v, AS_F32, B, H, Sq, Skv, 40, qs40, ks40, r.get(), P, 0.15f, (float*)out,
                          (float*)lse, nullptr) == AS_OK);
  CHECK(strcmp(stub::last.kind, "attn_f32") == 0 && stub::last.attn.n_qtiles == 5);
  CHECK(as_partition_attn_states(q, k, v, AS_F32, B, H, Sq, Skv, 40, qs40, ks40, r.get(), P, 0.15f, AS_FP8_E4M3, out,
                                 (float*)lse, nullptr) == AS_ERR_UNSUPPORTED);

  // grouped: the empty partition (2 of the 7) is packed out, its LSE filled with -inf
  {
    const std::vector<int32_t> gs = {0, 3, 3, 7};
    auto starts = ranges(gs);
    float* part = (float*)fake(0x70000000);
    stub::fills.clear();
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    starts.get(), 3, 0.088f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_OK);
    const as::AttnArgs& g = stub::last.attn;
    CHECK(strcmp(stub::last.kind, "attn_grouped") == 0 && g.G == 3 && g.P == 6);
    CHECK(g.group_starts[0] == 0 && g.group_starts[1] == 2 && g.group_starts[2] == 2 && g.group_starts[3] == 6);
    const int expect_index[6] = {0, 1, 3, 4, 5, 6};
    for (int i = 0; i < 6; ++i) {
      CHECK(g.part_index[i] == expect_index[i]);
      CHECK(g.ranges[2 * i] == flat[2 * expect_index[i]] && g.ranges[2 * i + 1] == flat[2 * expect_index[i] + 1]);
    }
    CHECK(stub::fills.size() == 1 && stub::fills[0].p == part + 2 * B * H * Sq && stub::fills[0].n == B * H * Sq);
    // group_starts not running from 0 to P, decreasing, G out of range, half a fold
    const std::vector<int32_t> bad1 = {0, 3, 6}, bad2 = {0, 4, 3, 7}, bad3 = {1, 7};
    auto b1 = ranges(bad1), b2 = ranges(bad2), b3 = ranges(bad3);
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    b1.get(), 2, 0.1f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_ERR_INVALID_ARG);
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    b2.get(), 3, 0.1f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_ERR_INVALID_ARG);
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    b3.get(), 1, 0.1f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_ERR_INVALID_ARG);
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    starts.get(), 0, 0.1f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_ERR_INVALID_ARG);
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    starts.get(), 3, 0.1f, (const float*)fake(0x60000000), nullptr, (float*)out,
                                    (float*)lse, part, nullptr) == AS_ERR_INVALID_ARG);
    CHECK(as_partition_attn_grouped(q, k, v, AS_F32, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    starts.get(), 3, 0.1f, nullptr, nullptr, (float*)out, (float*)lse, part,
                                    nullptr) == AS_ERR_INVALID_ARG);
    // the fold state overlapping an output
    CHECK(as_partition_attn_grouped(q, k, v, AS_BF16, nullptr, nullptr, nullptr, B, H, Sq, Skv, D, qs, ks, r.get(), P,
                                    starts.get(), 3, 0.1f, (const float*)out, (const float*)fake(0x61000000),
                                    (float*)out, (float*)lse, part, nullptr) == AS_ERR_INVALID_ARG);
  }

  // invalid: every one returns before any launch
  stub::last.kind = "";
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, -1.f, (float*)out, (float*)lse,
                          nullptr) == AS_ERR_INVALID_ARG);
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, NAN, (float*)out, (float*)lse,
                          nullptr) == AS_ERR_INVALID_ARG);
  // P beyond the maximum with a maximal-size range array: nothing past it is read
  std::vector<int32_t> many(2 * AS_MAX_PARTITIONS, 0);
  auto rm = ranges(many);
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, rm.get(), AS_MAX_PARTITIONS + 1, 0.1f,
                          (float*)out, (float*)lse, nullptr) == AS_ERR_INVALID_ARG);
  // sizes whose products overflow 64 bits
  CHECK(as_partition_attn(q, k, v, AS_BF16, INT64_MAX, INT64_MAX, Sq, Skv, D, qs, ks, r.get(), P, 0.1f, (float*)out,
                          (float*)lse, nullptr) == AS_ERR_UNSUPPORTED);
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, INT64_MAX, Skv, D, qs, ks, r.get(), P, 0.1f, (float*)out,
                          (float*)lse, nullptr) == AS_ERR_UNSUPPORTED);
  const int64_t huge[3] = {INT64_MAX - 7, INT64_MAX - 7, INT64_MAX - 7};
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, huge, ks, r.get(), P, 0.1f, (float*)out, (float*)lse,
                          nullptr) != AS_OK);
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, huge, r.get(), P, 0.1f, (float*)out, (float*)lse,
                          nullptr) != AS_OK);
  // overlapping outputs
  CHECK(as_partition_attn(q, k, v, AS_BF16, B, H, Sq, Skv, D, qs, ks, r.get(), P, 0.1f, (float*)q, (float*)lse,
                          nullptr) == AS_ERR_INVALID_ARG);
  CHECK(strcmp(stub::last.kind, "") == 0);
}

void merge_calls() {
  const int64_t rows = 1000, D = 128;
  for (int n : {1, 5, AS_MAX_MERGE}) {
    // pointer lists of exactly n entries
    std::unique_ptr<const float*[]> outs(new const float*[n]), lses(new const float*[n]);
    for (int i = 0; i < n; ++i) {
      outs[i] = (const float*)fake(0x10000000 + (uintptr_t)i * 0x100000);
      lses[i] = (const float*)fake(0x80000000 + (uintptr_t)i * 0x10000);
    }
    CHECK(as_merge(n, outs.get(), lses.get(), rows, D, (float*)fake(0x90000000), (float*)fake(0xa0000000),
                   nullptr) == AS_OK);
    CHECK(strcmp(stub::last.kind, "merge") == 0 && stub::last.merge.n == n && stub::last.merge.rows == rows);
    for (int i = 0; i < n; ++i) CHECK(stub::last.merge.outs[i] == outs[i] && stub::last.merge.lses[i] == lses[i]);
    std::unique_ptr<const void*[]> vouts(new const void*[n]);
    for (int i = 0; i < n; ++i) vouts[i] = outs[i];
    CHECK(as_merge_states(n, vouts.get(), lses.get(), AS_BF16, rows, D, AS_F32, fake(0x90000000),
                          (float*)fake(0xa0000000), nullptr) == AS_OK);
    CHECK(stub::last.merge.in_kind == 1 && stub::last.merge.out_kind == 0);
    CHECK(as_merge_states(n, vouts.get(), lses.get(), AS_FP8_E4M3, rows, D, AS_FP8_E4M3, fake(0x90000000),
                          (float*)fake(0xa0000000), nullptr) == AS_OK);
    CHECK(stub::last.merge.in_kind == 2 && stub::last.merge.out_kind == 2 &&
          stub::last.merge.payload_bytes == (int64_t)as_state_bytes(AS_FP8_E4M3, rows, D));
    // n one beyond the list: refused before reading it
    CHECK(as_merge(n + AS_MAX_MERGE, outs.get(), lses.get(), rows, D, (float*)fake(0x90000000),
                   (float*)fake(0xa0000000), nullptr) == AS_ERR_INVALID_ARG);
  }
  const float* one[1] = {(const float*)fake(0x10000000)};
  const float* onel[1] = {(const float*)fake(0x20000000)};
  CHECK(as_merge(1, one, onel, INT64_MAX, D, (float*)fake(0x90000000), (float*)fake(0xa0000000), nullptr) ==
        AS_ERR_UNSUPPORTED);
  CHECK(as_merge(1, one, onel, rows, D, (float*)fake(0x10000000 + 0x1000), (float*)fake(0xa0000000), nullptr) ==
        AS_ERR_INVALID_ARG);
  // group-wise composition
  CHECK(as_compose_groups(fake(0x10000000), (const float*)fake(0x80000000), AS_BF16, 32, rows, D, 4, AS_BF16,
                          fake(0x90000000), (float*)fake(0xa0000000), nullptr) == AS_OK);
  CHECK(stub::last.merge.group == 4 && stub::last.merge.n == 32);
  CHECK(as_compose_groups(fake(0x10000000), (const float*)fake(0x80000000), AS_FP8_E4M3, 32, rows, D, 4, AS_F32,
                          fake(0x90000000), (float*)fake(0xa0000000), nullptr) == AS_OK);
  CHECK(stub::last.merge.in_kind == 2 && stub::last.merge.out_kind == 0);
  // fp8 states need D in {32, 64, 128, 256}
  CHECK(as_compose_groups(fake(0x10000000), (const float*)fake(0x80000000), AS_FP8_E4M3, 32, rows, 96, 4, AS_F32,
                          fake(0x90000000), (float*)fake(0xa0000000), nullptr) == AS_ERR_UNSUPPORTED);
  CHECK(as_compose_groups(fake(0x10000000), (const float*)fake(0x80000000), AS_BF16, 32, INT64_MAX / 2, D, 4,
                          AS_BF16, fake(0x90000000), (float*)fake(0xa0000000), nullptr) == AS_ERR_UNSUPPORTED);
}

void contribution_and_planner_calls() {
  const int32_t P = 32;
  const int64_t rows = 24 * 3840, rpg = 3840;
  const size_t ws = as_partition_contribution_workspace_size(P, rows, rpg);
  CHECK(ws == (size_t)24 * 15 * 32 * 4);
  CHECK(as_partition_contribution_workspace_size(P, INT64_MAX, 1) == 0);
  CHECK(as_partition_contribution((const float*)fake(0x10000000), P, rows, rpg, (float*)fake(0x20000000),
                                  (float*)fake(0x30000000), fake(0x40000000), ws, nullptr) == AS_OK);
  CHECK(strcmp(stub::last.kind, "contribution") == 0 && stub::last.contrib.chunks_per_group == 15);
  CHECK(stub::last.contrib.partial == (float*)fake(0x40000000));
  CHECK(as_partition_contribution_noalloc((const float*)fake(0x10000000), P, rows, rpg, nullptr,
                                          (float*)fake(0x30000000), nullptr) == AS_OK);
  CHECK(stub::last.contrib.partial == (float*)stub::kScratchAddress && stub::last.contrib.weights == nullptr);
  CHECK(as_partition_contribution_noalloc((const float*)fake(0x10000000), 256, 256 * 1025, 256, nullptr,
                                          (float*)fake(0x30000000), nullptr) == AS_ERR_INVALID_ARG);
  CHECK(as_partition_contribution((const float*)fake(0x10000000), P, INT64_MAX - 1, 1, (float*)fake(0x20000000),
                                  nullptr, nullptr, 0, nullptr) == AS_ERR_UNSUPPORTED);

  const int64_t n = rows * 128;
  const size_t nws = as_state_norms_workspace_size(P, n);
  CHECK(nws > 0 && as_state_norms_workspace_size(P, INT64_MAX - 3) == 0);
  CHECK(as_state_norms((const float*)fake(0x100000000), (const float*)fake(0x200000000), P, n,
                       (float*)fake(0x10000000), fake(0x20000000), nws, nullptr) == AS_OK);
  CHECK(strcmp(stub::last.kind, "norms") == 0 && stub::last.norms.chunks * stub::last.norms.chunk >= n);
  CHECK(as_state_norms((const float*)fake(0x100000000), nullptr, P, INT64_MAX - 3, (float*)fake(0x10000000),
                       fake(0x20000000), nws, nullptr) != AS_OK);

  float* f = (float*)fake(0x10000000);
  int32_t* c = (int32_t*)fake(0x20000000);
  CHECK(as_planner_decide(f, f + 64, f + 128, f + 192, P, 16, 4, 0.5f, f + 256, f + 320, f + 384, c, c + 64,
                          nullptr) == AS_OK);
  CHECK(strcmp(stub::last.kind, "decide") == 0 && stub::last.plan.group == 4);
  CHECK(as_planner_decide(f, f + 64, f + 128, f + 192, P, 16, INT32_MAX, 0.5f, f + 256, f + 320, f + 384, c, c + 64,
                          nullptr) == AS_OK);
  CHECK(stub::last.plan.group == P);
  CHECK(as_planner_decide(f, f + 64, f + 128, f + 192, P, 16, 4, 0.5f, f + 8, f + 320, f + 384, c, c + 64,
                          nullptr) == AS_ERR_INVALID_ARG);
  CHECK(as_planner_epsilon(f, f + 64, P, 16, 4, 0.5f, f + 128, nullptr) == AS_OK);
  CHECK(as_planner_epsilon(f, f + 64, P, 16, INT32_MAX, 0.5f, f + 128, nullptr) == AS_OK);
  CHECK(as_planner_epsilon(f, f + 64, P, 16, 4, 0.5f, f + 3, nullptr) == AS_ERR_INVALID_ARG);
}

}  // namespace

int main() {
  for (int s = -1; s <= 4; ++s) CHECK(as_status_string((as_status)s) != nullptr);
  attn_calls();
  merge_calls();
  contribution_and_planner_calls();
  CHECK(as_last_error() != nullptr);
  printf("abi sanitize ok\n");
  return 0;
}
