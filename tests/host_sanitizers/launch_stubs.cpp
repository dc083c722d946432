// launch_stubs.cpp -- stand-ins for the kernel launchers of the library, for the
// sanitizer build of the host code: each counts the call and refuses it with
// hipErrorInvalidDeviceFunction, so no kernel is ever enqueued.
#include <hip/hip_runtime_api.h>

#include <atomic>

#include "forge_internal.h"

namespace {
std::atomic<int> g_launches{0};
int refuse() {
  g_launches.fetch_add(1);
  return (int)hipErrorInvalidDeviceFunction;
}
}  // namespace

namespace forge {
int launch_fused_step(int, int, int, int, const GemmArgs&, const EpiArgs&, void*) { return refuse(); }
int launch_wgrad_gemm(int, const GemmArgs&, float*, void*) { return refuse(); }
int launch_optimizer(int, int, int, const float*, int64_t, const EpiArgs&, void*) { return refuse(); }
int launch_dgrad(const void*, const void*, void*, int64_t, int64_t, int64_t, void*) { return refuse(); }
int launch_backward_step(int, int, const GemmArgs&, const EpiArgs&, const void*, void*, int*, void*) {
  return refuse();
}
int64_t backward_workspace_words(int64_t K) { return 26 + K / 128; }
int backward_scratch(int** out) {
  *out = nullptr;
  return refuse();
}
}  // namespace forge

extern "C" int forge_stub_launches(void) { return g_launches.load(); }
