// forge_backward.hip -- the backward step of a linear layer in one launch: dX = dY W with the
// weight as it was before the step, and the fused step of W (FORGE explainer, gist.science,
// Technical Summary section 2 "Core Mechanism", and section 5, limitations: the input gradient
// must be read before the weight is updated).
//
// One grid of 4-wave workgroups, two per CU, as many workgroups as work items.  The items come
// in three phases: the 256-token x 128-column dX tiles, then the fused step's 256 x 128 tiles,
// then its 128 x 128 half tiles (the layout of the 256 x 128 path, forge_plan.h).  Each phase
// has 8 queues, one per XCD slot (blockIdx mod 8, the XCD a workgroup is dispatched to): the
// k-th item of queue q is the tile that workgroup q + 8 k takes in the separate dgrad and step
// launches, so each XCD's L2 sees the same tile walk as there.  A workgroup starts with its own
// queue and moves on to the others when it is empty, so no item depends on where or in which
// order workgroups are dispatched.
// A dX tile of column block kb reads W[:, kb] in its contraction and then counts itself done in
// that column block's counter.  A step tile of column block kb contracts dY and X first and,
// before its update writes W, waits until all of kb's dX tiles are done.  The wait always ends:
// a workgroup takes a step tile only after it has seen every dX queue empty, so every dX tile
// is already held by a running workgroup, and dX tiles wait for nothing.  The wait is still
// bounded: past the bound the workgroup raises the error word, skips its update and exits, so
// no wave is left waiting.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "forge_dgrad.h"
#include "forge_fused2.h"

// The counters of the allocation-free entry point: one array per device, for the life of the
// process (kBackwardScratchWords words).  Host code never passes this name to a kernel: it is
// a host-side stand-in; backward_scratch() resolves the device address.
static __device__ __align__(256) int scratch[forge::kBackwardScratchWords];

namespace forge {

// Workspace words: [1] the error word; [2 + 8 p + q] claims made on queue q of phase p
// (0: dX tiles, 1: full step tiles, 2: half step tiles; forge_plan.h); [26 + kb] dX tiles of
// column block kb that have finished reading W.
enum : int { BWD_ERROR = 1, BWD_QUEUES = 2, BWD_DONE = BWD_QUEUES + plan::kPhases * plan::kQueues };
constexpr int kClaimAttempts = 64;

// Wave 0 claims the workgroup's item: phase and index within the phase (-1 if none is left,
// which only overlapping calls on one workspace can cause).  One snapshot of the 24 queue
// counters (lane l reads counter l) picks the queue (plan::pick_queue); an atomic add claims an
// item there, or, if others used up that queue meanwhile, the snapshot is taken again.  Counters
// only grow, so a queue seen used up stays so.
__device__ __forceinline__ void claim_item(const BackwardArgs& b, const GemmArgs& g, int& phase, int& index) {
  const int lane = (int)(threadIdx.x & 63), q0 = (int)(blockIdx.x & (plan::kQueues - 1));
  const plan::BackwardItems it = plan::backward_items(g, b.nbT);
  const int ln = plan::phase_items(it, lane / plan::kQueues);
  const bool counter_lane = lane < plan::kPhases * plan::kQueues;
  phase = -1;
  index = -1;
  for (int attempt = 0; attempt < kClaimAttempts; ++attempt) {
    int c = 0;
    if (counter_lane) c = __hip_atomic_load(b.ctr + BWD_QUEUES + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t open = (uint32_t)__ballot(counter_lane && c < plan::queue_size(ln, lane % plan::kQueues));
    int p, q;
    if (!plan::pick_queue(open, q0, p, q)) return;
    int k = 0;
    if (lane == 0) k = atomicAdd(b.ctr + BWD_QUEUES + plan::kQueues * p + q, 1);
    k = __shfl(k, 0);
    const int item = plan::claimed_item(plan::phase_items(it, p), q, k);
    if (item >= 0) {
      phase = p;
      index = item;
      return;
    }
  }
}

// Waits (one thread) until *p >= want; false once `limit` polls have gone by.
__device__ __forceinline__ bool wait_at_least(const int* p, int want, int limit) {
  for (int i = 0;; ++i) {
    if (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
    if (i >= limit) return false;
    __builtin_amdgcn_s_sleep(4);
  }
}

template <int ST, int OPT>
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void backward_step_kernel(GemmArgs g, EpiArgs e, BackwardArgs b) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  __shared__ int phase_s, index_s, ready_s;
  if (threadIdx.x < 64) {
    int p, i;
    claim_item(b, g, p, i);
    if (threadIdx.x == 0) {
      phase_s = p;
      index_s = i;
      if (p < 0) atomicOr(b.ctr + BWD_ERROR, 2);
    }
  }
  __syncthreads();
  const int phase = phase_s, index = index_s;
  if (phase < 0) return;
  if (phase == 0) {
    int tb, kb;
    plan::tile_coords_at(index, b.nbT, g.nbk, tb, kb);
    dgrad_tile(static_cast<const uint16_t*>(g.dY), b.W_old, b.dX, g.T, g.N, g.K, (int64_t)tb * ml2::BM,
               kb * ml2::BN, smem, [&] {
                 // every wave's reads of W[:, kb] have completed (the contraction ended with a barrier)
                 if (threadIdx.x == 0)
                   __hip_atomic_fetch_add(b.ctr + BWD_DONE + kb, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
               });
    return;
  }
  int n0, k0;
  if (phase == 1) plan::full_tile(g, index, n0, k0);
  else plan::half_tile(g, index, n0, k0);
  const int kb = k0 / ml2::BN;
  auto before_update = [&]() -> bool {
    if (threadIdx.x == 0) {
      const bool ok = wait_at_least(b.ctr + BWD_DONE + kb, b.nbT, b.spin_limit);
      if (!ok) atomicOr(b.ctr + BWD_ERROR, 1);
      ready_s = ok ? 1 : 0;
    }
    __syncthreads();
    return ready_s != 0;
  };
  if (phase == 1) fused_full_tile_at<FORGE_W_BF16, ST, OPT>(g, e, smem, n0, k0, before_update);
  else fused_half_tile_at<FORGE_W_BF16, ST, OPT>(g, e, smem, n0, k0, before_update);
}

__global__ __launch_bounds__(256) void clear_words_kernel(int* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += 256) p[i] = 0;
}

using BackwardFn = void (*)(GemmArgs, EpiArgs, BackwardArgs);

template <int ST>
static BackwardFn backward_for(int opt) {
  switch (opt) {
#define FORGE_CASE(O) \
  case O: return backward_step_kernel<ST, O>;
    FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
  }
  return nullptr;
}

int64_t backward_workspace_words(int64_t K) { return BWD_DONE + K / ml2::BN; }

namespace {
std::mutex g_scratch_mu;
std::atomic<int*> g_scratch[64];
}  // namespace

int backward_scratch(int** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return (int)err;
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  int* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));  // with device `dev` current
      if (err != hipSuccess) return (int)err;
      p = static_cast<int*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return (int)hipSuccess;
}

int launch_backward_step(int s_type, int opt, const GemmArgs& g_in, const EpiArgs& e, const void* W_old, void* dX,
                         int* ctr, void* stream) {
  BackwardFn fn = s_type == FORGE_S_F32  ? backward_for<FORGE_S_F32>(opt)
                  : s_type == FORGE_S_Q8 ? backward_for<FORGE_S_Q8>(opt)
                                         : backward_for<FORGE_S_Q8D>(opt);
  if (!fn) return (int)hipErrorInvalidValue;
  GemmArgs g = plan::whole_dma(g_in);
  const int cus = slots_on_current_device() / 2;
  const unsigned n_step = plan::plan_split(g, 2 * cus);
  BackwardArgs b{};
  b.W_old = static_cast<const uint16_t*>(W_old);
  b.dX = static_cast<uint16_t*>(dX);
  b.ctr = ctr;
  b.nbT = (int)((g.T + ml2::BM - 1) / ml2::BM);
  b.n_dgrad = b.nbT * g.nbk;
  b.spin_limit = kBackwardSpinLimit;
  const int words = (int)backward_workspace_words(g.K);
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, ctr, words);
  const unsigned grid = (unsigned)b.n_dgrad + n_step;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(ml2::THREADS), 0, (hipStream_t)stream, g, e, b);
  return (int)hipGetLastError();
}

}  // namespace forge
