// Recorder shared by the launcher stand-ins and the sanitizer driver.
#pragma once
#include <vector>

#include "as_internal.h"

namespace stub {
constexpr uintptr_t kScratchAddress = 0x7000000;
struct Record {
  const char* kind = "";
  as::AttnArgs attn{};
  as::MergeArgs merge{};
  as::ContribArgs contrib{};
  as::NormArgs norms{};
  as::PlanArgs plan{};
};
extern Record last;
struct Fill {
  float* p;
  int64_t n;
};
extern std::vector<Fill> fills;   // -inf fills of empty partitions' LSE
}  // namespace stub
