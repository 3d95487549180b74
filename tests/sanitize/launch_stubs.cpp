// Host-only stand-ins for the kernel launchers of the attention-state library, so that
// the C ABI layer (api.hip, compiled here as plain C++) can run under AddressSanitizer
// and UndefinedBehaviorSanitizer without a GPU. Each stand-in records the argument
// block it was given; nothing is launched.
#include "launch_stubs.h"

namespace stub {
Record last;
std::vector<Fill> fills;
}

namespace as {

int attn_bf16_rows_per_block(int) { return 256; }
int attn_f32_rows_per_block(int) { return 64; }

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "attn_bf16";
  stub::last.attn = a;
  return hipSuccess;
}
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "attn_fp8";
  stub::last.attn = a;
  return hipSuccess;
}
hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "attn_grouped";
  stub::last.attn = a;
  return hipSuccess;
}
hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t) {
  stub::fills.push_back({p, n});
  return hipSuccess;
}
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "attn_f32";
  stub::last.attn = a;
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "merge";
  stub::last.merge = a;
  return hipSuccess;
}
hipError_t launch_contribution(const ContribArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "contribution";
  stub::last.contrib = a;
  return hipSuccess;
}
hipError_t launch_state_norms(const NormArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "norms";
  stub::last.norms = a;
  return hipSuccess;
}
hipError_t launch_planner_decide(const PlanArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "decide";
  stub::last.plan = a;
  return hipSuccess;
}
hipError_t launch_planner_epsilon(const PlanArgs& a, hipStream_t) {
  stub::last = stub::Record();
  stub::last.kind = "epsilon";
  stub::last.plan = a;
  return hipSuccess;
}
hipError_t contribution_scratch(float** ptr) {
  *ptr = reinterpret_cast<float*>(stub::kScratchAddress);
  return hipSuccess;
}

}  // namespace as

const char* hipGetErrorString(hipError_t) { return "stub"; }
