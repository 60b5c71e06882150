// Kernel launch helper shared by the launchers: records the measurement
// hook's events around one launch when the hook names that kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <mutex>
#include <set>

#include "qmoe_internal.h"

namespace qmoe {

// Raises a kernel's dynamic-LDS limit to the device maximum, once per kernel
// per process (the attribute is an upper bound, the launch passes the size).
inline hipError_t ensure_dyn_lds(const void* fn) {
  static std::mutex mu;
  static std::set<const void*> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count(fn)) return hipSuccess;
  int dev = 0, max_lds = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e == hipSuccess) e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
  if (e == hipSuccess) done.insert(fn);
  return e;
}

// Runs launch(start, stop): the launch passes the two events to
// hipExtLaunchKernel, which records the kernel dispatch's own start and end
// times in them (null events: a plain launch).  The events come from a
// pending moe_profile_next_launch request for this kernel, which is consumed.
template <typename F>
hipError_t launch_timed(int kernel_id, hipStream_t s, F&& launch) {
  (void)s;
  ProfileHook& hk = profile_hook();
  int slot = -1;
  for (int i = 0; i < hk.n; ++i)
    if (hk.kernel_id[i] == kernel_id) {
      slot = i;
      break;
    }
  hipEvent_t start = nullptr, stop = nullptr;
  if (slot >= 0) {
    start = (hipEvent_t)hk.start[slot];
    stop = (hipEvent_t)hk.stop[slot];
    for (int i = slot + 1; i < hk.n; ++i) {   // consume the entry
      hk.kernel_id[i - 1] = hk.kernel_id[i];
      hk.start[i - 1] = hk.start[i];
      hk.stop[i - 1] = hk.stop[i];
    }
    --hk.n;
  }
  launch(start, stop);
  return hipGetLastError();
}

}  // namespace qmoe
