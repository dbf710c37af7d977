// Kernel launch with the optional per-kernel timing hook of the ABI
// (tp_profile_begin / tp_profile_end): while a caller has armed it on this
// thread, each launch records the caller's hipEvent pair around the kernel
// (hipExtLaunchKernelGGL) and remembers a static label for it.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

namespace tpk {

struct ProfileState {
  hipEvent_t const* start = nullptr;
  hipEvent_t const* stop = nullptr;
  int capacity = 0;
  int count = 0;
  std::vector<const char*> labels;   // one per event pair, sized at arming
  std::string only;                  // if not empty: the one label that records events
};

ProfileState& profile_state();   // thread-local, defined in tp_shard.cpp

template <class F, class... Args>
inline hipError_t launch(const char* label, F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  ProfileState& ps = profile_state();
  if (ps.start && ps.count < ps.capacity && (ps.only.empty() || ps.only == label)) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ps.start[ps.count], ps.stop[ps.count], 0, args...);
    ps.labels[ps.count] = label;
    ++ps.count;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  }
  return hipGetLastError();
}

}  // namespace tpk
