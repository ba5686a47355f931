// Opt-in per-kernel timing with HIP events (tree_attn_profile_* in the ABI).
#pragma once
#include <hip/hip_runtime.h>

namespace ta {

// Brackets the kernels launched during its lifetime with HIP events on
// `stream` when profiling is enabled; does nothing otherwise.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

}  // namespace ta
