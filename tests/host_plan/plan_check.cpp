// plan_check.cpp -- host check of the launch plans and tile mappings in forge_plan.h, the code
// the kernels and launchers run: for many weight shapes, token counts, CU counts, input types
// and both the fused step and the GEMM, every 64 x 64 block of W must be covered by exactly
// one workgroup, every tile must lie inside W, and every grid must be non-empty and exact.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "forge_plan.h"

using namespace forge;
using namespace forge::plan;

static int g_fail = 0;

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      std::fprintf(stderr, __VA_ARGS__);  \
      std::fprintf(stderr, "\n");         \
      ++g_fail;                           \
      return;                             \
    }                                     \
  } while (0)

static void check(int in_type, long N, long K, long T, int cus, int fused) {
  GemmArgs g{};
  g.N = N;
  g.K = K;
  g.T = T;
  Launch L[2];
  const int n = plan_launches(in_type, g, cus, fused, L);
  CHECK(n >= 1 && n <= 2, "N=%ld K=%ld: %d launches", N, K, n);
  std::vector<int> hit((size_t)(N / 64) * (size_t)(K / 64), 0);
  // coverage is counted on 64 x 64 blocks (the smallest tile)
  auto mark = [&](long n0, long k0, long rows, long cols) -> bool {
    if (n0 < 0 || k0 < 0 || n0 % 64 || k0 % 64 || n0 + rows > N || k0 + cols > K) return false;
    for (long r = n0 / 64; r < (n0 + rows) / 64; ++r)
      for (long c = k0 / 64; c < (k0 + cols) / 64; ++c) ++hit[(size_t)r * (size_t)(K / 64) + (size_t)c];
    return true;
  };
  for (int i = 0; i < n; ++i) {
    const GemmArgs& a = L[i].g;
    CHECK(L[i].grid > 0, "N=%ld K=%ld T=%ld cus=%d: empty grid", N, K, T, cus);
    for (unsigned b = 0; b < L[i].grid; ++b) {
      int n0 = 0, k0 = 0;
      long rows = 0, cols = 0;
      switch (L[i].kind) {
        case LAUNCH_WIDE:
          if (in_type == FORGE_IN_BF16) {
            CHECK(fused && a.kb_split % 2 == 0 && a.hk % 2 == 0 && a.nfull == a.nbn * (a.kb_split / 2) &&
                      L[i].grid == (unsigned)(a.nfull + a.hn * a.hk) && a.nfront >= 0 && a.nfront <= a.hn * a.hk,
                  "bad wide launch");
            const bool half = wide_item(a, (int)b, n0, k0);
            rows = half ? kHalfRows : kRows, cols = 2 * kCols;
          } else {
            CHECK(fused && a.nbk % 2 == 0 && a.hn == 0 && L[i].grid == (unsigned)(a.nbn * (a.nbk / 2)),
                  "bad wide launch");
            wide_tile(a, (int)b, n0, k0);
            rows = kRows, cols = 2 * kCols;
          }
          break;
        case LAUNCH_V2:
          if ((int)b < a.nfull) full_tile(a, (int)b, n0, k0), rows = kRows, cols = kCols;
          else half_tile(a, (int)b - a.nfull, n0, k0), rows = kHalfRows, cols = kCols;
          break;
        case LAUNCH_V8:
          CHECK(L[i].grid == (unsigned)(a.nbn * a.nbk), "bad fp8 grid");
          tile8(a, (int)b, n0, k0);
          rows = kRows, cols = kCols;
          break;
        default: {
          const int t = L[i].tile;
          CHECK(t == 128 || (t == 64 && in_type == FORGE_IN_F32), "bad small tile %d", t);
          const int nbN = (int)(N / t), nbK = (int)(K / t);
          CHECK(L[i].grid == (unsigned)(nbN * nbK), "bad small grid");
          int nb, kb;
          tile_coords_at((int)b, nbN, nbK, nb, kb);
          n0 = nb * t, k0 = kb * t, rows = t, cols = t;
        }
      }
      CHECK(mark(n0, k0, rows, cols), "N=%ld K=%ld T=%ld cus=%d launch %d kind %d wg %u: tile (%d, %d) outside W", N,
            K, T, cus, i, L[i].kind, b, n0, k0);
    }
  }
  for (size_t j = 0; j < hit.size(); ++j)
    CHECK(hit[j] == 1, "N=%ld K=%ld T=%ld cus=%d in=%d fused=%d: block (%zu, %zu) covered %d times", N, K, T, cus,
          in_type, fused, j / (size_t)(K / 64), j % (size_t)(K / 64), hit[j]);
}

int main() {
  // the workloads' layers, the test shapes and ragged / odd block counts
  const long shapes[][2] = {{4096, 14336}, {14336, 4096}, {4096, 4096}, {1024, 4096}, {6144, 4096}, {4096, 4224},
                            {2048, 4096},  {5120, 5120},  {17408, 5120}, {5120, 17408}, {1024, 5120}, {256, 384},
                            {256, 256},    {768, 2048},   {12288, 4096}, {6144, 4224}, {2048, 8192},  {512, 33280},
                            {128, 128},    {384, 640},    {256, 128}};
  const long Ts[] = {64, 200, 4096, 8192, 8193, 16384};
  const int cuss[] = {256, 304, 80, 1};
  const int ins[] = {FORGE_IN_F32, FORGE_IN_BF16, FORGE_IN_FP8};
  int cases = 0;
  for (const auto& s : shapes)
    for (long T : Ts)
      for (int cus : cuss)
        for (int in : ins)
          for (int fused = 0; fused < 2; ++fused) {
            check(in, s[0], s[1], T, cus, fused);
            ++cases;
          }
  // the wide plans taken at 256 CUs for the Llama-3.1-8B shapes at T = 8192: bf16 puts the
  // whole weight in one launch with one round of half-wide tiles (the last 8 row blocks of
  // gate/up, the last 8 256-column blocks of down_proj), fp8 keeps whole rounds of wide tiles
  // on part of the weight
  GemmArgs g{};
  g.T = 8192;
  g.N = 14336;
  g.K = 4096;
  const WidePlan a = plan_wide(g, 256, true), a8 = plan_wide(g, 256, false);
  g.N = 4096;
  g.K = 14336;
  const WidePlan b = plan_wide(g, 256, true), b8 = plan_wide(g, 256, false);
  if (!(a.hr == 8 && a.hc == 0 && b.hc == 8 && b.hr == 0 && a8.nw == 48 && a8.kw == 0 && b8.kw == 48 && b8.nw == 0)) {
    std::fprintf(stderr, "unexpected wide plans: gate (%d, %d, %d), down (%d, %d, %d)\n", a.hr, a8.nw, a8.kw, b.hc,
                 b8.kw, b8.nw);
    ++g_fail;
  }
  // down_proj at T = 4096 and 8192: one launch of 768 wide tiles between two runs of 128
  // half-wide tiles; at T = 4096 a weight whose wide tiles fill whole rounds (4096 x 4096), and
  // fp8 inputs, stay on the 256 x 128 path
  for (long T : {4096L, 8192L}) {
    Launch L[2];
    g.T = T;
    g.N = 4096;
    g.K = 14336;
    int n = plan_launches(FORGE_IN_BF16, g, 256, 1, L);
    if (!(n == 1 && L[0].kind == LAUNCH_WIDE && L[0].g.nfull == 768 && L[0].g.hn * L[0].g.hk == 256 &&
          L[0].grid == 1024 && L[0].g.nfront == 128)) {
      std::fprintf(stderr, "unexpected down_proj wide launch at T = %ld\n", T);
      ++g_fail;
    }
    n = plan_launches(FORGE_IN_FP8, g, 256, 1, L);
    if (T == 4096 && !(n == 1 && L[0].kind == LAUNCH_V8)) {
      std::fprintf(stderr, "fp8 down_proj at T = 4096 took wide tiles\n");
      ++g_fail;
    }
  }
  {
    Launch L[2];
    g.T = 4096;
    g.N = 4096;
    g.K = 4096;
    const int n = plan_launches(FORGE_IN_BF16, g, 256, 1, L);
    if (!(n == 1 && L[0].kind == LAUNCH_V2)) {
      std::fprintf(stderr, "4096 x 4096 at T = 4096 took wide tiles\n");
      ++g_fail;
    }
  }
  std::printf("plan_check: %d cases, %d failures\n", cases, g_fail);
  return g_fail ? 1 : 0;
}
