// queue_check.cpp -- host check of the work queues of the one-launch backward step, with the
// functions of forge_plan.h that the kernel runs (backward_items, queue_size, pick_queue,
// claimed_item) and the kernel's claim protocol: a workgroup takes one snapshot of the 24 claim
// counters, picks a queue from it, and claims with one atomic add, taking a new snapshot if the
// queue was used up meanwhile.  Workgroups start, snapshot and claim in a random interleaving.
// Checked, over many shapes, CU counts and interleavings:
//   * every item of every phase is claimed exactly once and every workgroup gets one item;
//   * no step item (phase 1 or 2) is claimed while a dX item (phase 0) is still unclaimed, which
//     is what makes the step tiles' waits finite;
//   * a workgroup needs few snapshots (the device gives up after 64);
//   * the claimed indices map to tiles that cover dX and W exactly once.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "forge_plan.h"

using namespace forge;
using namespace forge::plan;

static int g_fail = 0;

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      std::fprintf(stderr, __VA_ARGS__); \
      std::fprintf(stderr, "\n");        \
      ++g_fail;                          \
      return;                            \
    }                                    \
  } while (0)

struct Workgroup {
  int q0;
  int phase = -1, queue = -1;  // picked, not yet claimed
  int attempts = 0;
  bool done = false;
};

// One launch: grid workgroups claim the items of `it` in an interleaving drawn from `rng`.
static void simulate(const BackwardItems& it, std::mt19937& rng, std::vector<std::vector<int>>& claims,
                     int& max_attempts) {
  const int grid = it.dgrad + it.full + it.half;
  int counters[kPhases * kQueues] = {};
  claims.assign(kPhases, {});
  for (int p = 0; p < kPhases; ++p) claims[p].assign(phase_items(it, p), 0);
  std::vector<Workgroup> wgs;
  int started = 0, finished = 0, dgrad_claimed = 0;
  max_attempts = 0;
  std::vector<int> active;
  while (finished < grid) {
    // start a new workgroup (dispatch order: blockIdx order, XCD slot blockIdx mod 8), or step one
    if (started < grid && (active.empty() || rng() % 3 == 0)) {
      Workgroup w;
      w.q0 = started % kQueues;
      wgs.push_back(w);
      active.push_back(started++);
      continue;
    }
    const size_t pick = rng() % active.size();
    Workgroup& w = wgs[active[pick]];
    if (w.phase < 0) {  // snapshot
      uint32_t open = 0;
      for (int l = 0; l < kPhases * kQueues; ++l)
        if (counters[l] < queue_size(phase_items(it, l / kQueues), l % kQueues)) open |= 1u << l;
      int p, q;
      CHECK(pick_queue(open, w.q0, p, q), "workgroup %d found no open queue", active[pick]);
      CHECK(p >= 0 && p < kPhases && q >= 0 && q < kQueues && (open >> (kQueues * p + q) & 1u), "bad pick");
      w.phase = p;
      w.queue = q;
      ++w.attempts;
    } else {  // claim
      const int k = counters[kQueues * w.phase + w.queue]++;
      const int n = phase_items(it, w.phase);
      const int item = claimed_item(n, w.queue, k);
      if (item >= 0) {
        CHECK(item < n, "item %d of %d", item, n);
        if (w.phase > 0) CHECK(dgrad_claimed == it.dgrad, "step item claimed with dX items unclaimed");
        else ++dgrad_claimed;
        ++claims[w.phase][item];
        w.done = true;
        if (w.attempts > max_attempts) max_attempts = w.attempts;
        active[pick] = active.back();
        active.pop_back();
        ++finished;
      } else {
        w.phase = -1;  // used up meanwhile: take a new snapshot
      }
    }
  }
  for (int p = 0; p < kPhases; ++p)
    for (size_t i = 0; i < claims[p].size(); ++i)
      CHECK(claims[p][i] == 1, "phase %d item %zu claimed %d times", p, i, claims[p][i]);
  CHECK(max_attempts < 64, "a workgroup needed %d snapshots", max_attempts);
}

// The tiles the kernel takes for the claimed indices cover dX [T, K] and W [N, K] exactly once.
static void check_tiles(const GemmArgs& g, int nbT) {
  const BackwardItems it = backward_items(g, nbT);
  std::vector<int> dx((size_t)nbT * g.nbk, 0);
  for (int i = 0; i < it.dgrad; ++i) {
    int tb, kb;
    tile_coords_at(i, nbT, g.nbk, tb, kb);
    CHECK(tb >= 0 && tb < nbT && kb >= 0 && kb < g.nbk, "dX tile out of range");
    ++dx[(size_t)tb * g.nbk + kb];
  }
  for (int c : dx) CHECK(c == 1, "dX tile covered %d times", c);
  // W in 128 x 128 blocks
  std::vector<int> w((size_t)(g.N / 128) * (g.K / 128), 0);
  auto mark = [&](int n0, int k0, int rows) {
    for (int r = n0 / 128; r < (n0 + rows) / 128; ++r) ++w[(size_t)r * (g.K / 128) + k0 / 128];
  };
  for (int i = 0; i < it.full; ++i) {
    int n0, k0;
    full_tile(g, i, n0, k0);
    CHECK(n0 >= 0 && n0 + 256 <= g.N && k0 >= 0 && k0 + 128 <= g.K, "full tile out of W");
    mark(n0, k0, 256);
  }
  for (int i = 0; i < it.half; ++i) {
    int n0, k0;
    half_tile(g, i, n0, k0);
    CHECK(n0 >= 0 && n0 + 128 <= g.N && k0 >= 0 && k0 + 128 <= g.K, "half tile out of W");
    mark(n0, k0, 128);
  }
  for (int c : w) CHECK(c == 1, "W block covered %d times", c);
}

int main() {
  const long shapes[][2] = {{4096, 14336}, {14336, 4096}, {4096, 4096}, {1024, 4096}, {1024, 5120},
                            {256, 384},    {512, 1024},   {2048, 4224}, {256, 128},   {768, 640}};
  const long Ts[] = {0, 1, 200, 257, 4096, 8192};
  const int cuss[] = {256, 80, 3};
  std::mt19937 rng(12345);
  int cases = 0, worst = 0;
  std::vector<std::vector<int>> claims;
  for (const auto& s : shapes)
    for (long T : Ts)
      for (int cus : cuss) {
        GemmArgs g{};
        g.N = s[0];
        g.K = s[1];
        g.T = T;
        g = whole_dma(g);
        plan_split(g, 2 * cus);
        const int nbT = (int)((T + 255) / 256);
        check_tiles(g, nbT);
        const BackwardItems it = backward_items(g, nbT);
        // large launches once, small ones under several interleavings
        const int reps = it.dgrad + it.full + it.half > 20000 ? 1 : 4;
        for (int r = 0; r < reps; ++r) {
          int att = 0;
          simulate(it, rng, claims, att);
          if (att > worst) worst = att;
          ++cases;
        }
      }
  // pick_queue on its own: own queue first, then the next open one; earliest phase wins
  {
    int p, q;
    if (!(pick_queue(0x00FF00u, 3, p, q) && p == 1 && q == 3)) ++g_fail;
    if (!(pick_queue(1u << 5 | 1u << 1, 3, p, q) && p == 0 && q == 5)) ++g_fail;
    if (!(pick_queue(1u << 1 | 1u << 20, 6, p, q) && p == 0 && q == 1)) ++g_fail;
    if (pick_queue(0u, 0, p, q)) ++g_fail;
  }
  std::printf("queue_check: %d launches simulated, at most %d snapshots per workgroup, %d failures\n", cases, worst,
              g_fail);
  return g_fail ? 1 : 0;
}
