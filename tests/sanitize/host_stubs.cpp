// Stand-ins for the kernel launchers and for the one HIP runtime call the host API makes, so
// that libmixer's host code (argument validation, the Latin-square scheduler, the layer
// runner) builds with g++ under AddressSanitizer and UndefinedBehaviorSanitizer on a host
// without a GPU. Every launch is recorded for the driver to inspect; nothing touches a device.
#include <vector>

#include "kernels.h"

std::vector<mixer::PrefillLaunch> g_launches;
int g_ceiling_calls = 0;
int g_events = 0;

namespace mixer {

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t) {
  g_launches.push_back(a);
  return hipSuccess;
}

hipError_t launch_mfma_ceiling(const void*, int, float*, int, int, hipStream_t) {
  ++g_ceiling_calls;
  return hipSuccess;
}

}  // namespace mixer

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++g_events;
  return hipSuccess;
}
