// forge_measure.hip -- the shader-clock sampler declared in include/forge_measure.h.
#include <hip/hip_runtime.h>

#include "forge_measure.h"

namespace {

// One lane reads both counters, sleeps between real-time reads until `ticks` have passed (a
// wait bounded by real time, so the wave always ends), then stores the two differences.
__global__ __launch_bounds__(64) void clock_sampler_kernel(uint64_t ticks, uint64_t* out) {
  if (threadIdx.x != 0) return;
  const uint64_t r0 = wall_clock64(), c0 = clock64();
  uint64_t r = r0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(32);
    r = wall_clock64();
  }
  const uint64_t c1 = clock64();
  out[0] = c1 - c0;
  out[1] = r - r0;
}

double realtime_hz_current() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0.0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return 0.0;
  return 1e3 * (double)khz;
}

}  // namespace

extern "C" {

forge_status forge_clock_sample(double seconds, uint64_t* out, void* stream) {
  if (!out || !(seconds > 0.0 && seconds <= 10.0)) return FORGE_ERR_ARG;
  const double hz = realtime_hz_current();
  if (hz <= 0.0) return FORGE_ERR_DEVICE;
  const uint64_t ticks = (uint64_t)(seconds * hz);
  hipLaunchKernelGGL(clock_sampler_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ticks, out);
  return hipGetLastError() == hipSuccess ? FORGE_OK : FORGE_ERR_LAUNCH;
}

double forge_realtime_hz(void) { return realtime_hz_current(); }

}  // extern "C"
