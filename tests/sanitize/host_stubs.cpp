// Stand-ins for the kernel launchers and for the one HIP runtime call the host API makes, so
// that libmixer's host code (argument validation, the Latin-square scheduler, the layer
// runner) builds with g++ under AddressSanitizer and UndefinedBehaviorSanitizer on a host
// without a GPU. Every launch is recorded for the driver to inspect; nothing touches a device.
#include <vector>

#include "kernels.h"

std::vector<mixer::PrefillLaunch> g_launches;
int g_ceiling_calls = 0;
int g_events = 0;
// When >= 0: the launch with this index (counted from 0 across the run) is refused, as the
// runtime would refuse it, and not recorded.
long g_fail_launch_at = -1;
long g_launch_calls = 0;
// When >= 0: the event record with this index is refused.
long g_fail_event_at = -1;

namespace mixer {

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t) {
  if (g_launch_calls++ == g_fail_launch_at) return hipErrorLaunchFailure;
  g_launches.push_back(a);
  return hipSuccess;
}

hipError_t launch_mfma_ceiling(const void*, int, float*, int, int, hipStream_t) {
  ++g_ceiling_calls;
  return hipSuccess;
}

}  // namespace mixer

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  if (g_events == g_fail_event_at) return hipErrorInvalidHandle;
  ++g_events;
  return hipSuccess;
}
