// forge_plan.h -- how a weight is cut into workgroup tiles: the launch plans of the fused step
// and the GEMM, and the tile each workgroup takes.  Host and device share this code (the
// kernels map blockIdx to a tile with it, the launchers size their grids with it, and a host
// test checks with it that every element of W is covered exactly once).
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": one workgroup
// accumulates whole tiles of W over all tokens; the tile shape does not change the result.
#pragma once

#include <hip/hip_runtime.h>

#include "forge_internal.h"

namespace forge {
namespace plan {

constexpr int kRows = 256;      // full tile rows (n) on the LDS-DMA paths
constexpr int kCols = 128;      // tile columns (k); a wide tile spans two
constexpr int kHalfRows = 128;  // half tile rows
constexpr int kSmallTile = 128; // register-staged path: 128 x 128 tiles (64 x 64 for small fp32 layers)

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8), each
// with its own L2.  Give every XCD a contiguous run of tile ids, and inside a run walk the
// tiles in groups of 4 row blocks, so that concurrently running tiles share dY and X panels in
// their XCD's L2.  Maps b in [0, nbN nbK) to (nb, kb) one to one.
__host__ __device__ inline void tile_coords_at(int b, int nbN, int nbK, int& nb, int& kb) {
  const int nt = nbN * nbK;
  const int per = nt >> 3, rem = nt & 7, x = b & 7, loc = b >> 3;
  const int t = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + loc;
  constexpr int G = 4;
  const int group = G * nbK;
  const int gid = t / group, first = gid * G;
  const int gsz = (nbN - first) < G ? (nbN - first) : G;
  const int r = t - gid * group;
  nb = first + r % gsz;
  kb = r / gsz;
}

// ---- tile origins, per kind of workgroup (row n0 and column k0 of its first element)
// 256 x 128 tile b in [0, nfull) of a 256 x 128 launch (fused step or GEMM).
__host__ __device__ inline void full_tile(const GemmArgs& g, int b, int& n0, int& k0) {
  int nb, kb;
  tile_coords_at(b, g.nbn, g.kb_split, nb, kb);
  n0 = (g.nb_base + nb) * kRows;
  k0 = (g.kb_base + kb) * kCols;
}
// 128 x 128 half tile hb (the workgroups after nfull) of a 256 x 128 launch.
__host__ __device__ inline void half_tile(const GemmArgs& g, int hb, int& n0, int& k0) {
  int nb, kb;
  tile_coords_at(hb, 2 * g.nbn, g.nbk - g.kb_split, nb, kb);
  n0 = g.nb_base * kRows + nb * kHalfRows;
  k0 = (g.kb_base + g.kb_split + kb) * kCols;
}
// Workgroup b of a bf16 wide launch: the origin of its tile, and whether that tile is a
// 128 x 256 half-wide one (the first nfront workgroups and those after the nfull wide tiles)
// rather than 256 x 256 (columns k0 .. k0 + 255 either way).
__host__ __device__ inline bool wide_item(const GemmArgs& g, int b, int& n0, int& k0) {
  int nb, kb;
  const int w = b - g.nfront;
  if (w >= 0 && w < g.nfull) {
    tile_coords_at(w, g.nbn, g.kb_split / 2, nb, kb);
    n0 = (g.nb_base + nb) * kRows;
    k0 = (g.kb_base + 2 * kb) * kCols;
    return false;
  }
  tile_coords_at(w < 0 ? b : b - g.nfull, 2 * g.hn, g.hk / 2, nb, kb);
  n0 = g.h_nb * kRows + nb * kHalfRows;
  k0 = (g.h_kb + 2 * kb) * kCols;
  return true;
}
// 256 x 256 tile b of an fp8 wide launch (columns k0 .. k0 + 255).
__host__ __device__ inline void wide_tile(const GemmArgs& g, int b, int& n0, int& k0) {
  int nb, kb;
  tile_coords_at(b, g.nbn, g.nbk / 2, nb, kb);
  n0 = (g.nb_base + nb) * kRows;
  k0 = (g.kb_base + 2 * kb) * kCols;
}
// 256 x 128 tile b of an fp8 launch (no half tiles).
__host__ __device__ inline void tile8(const GemmArgs& g, int b, int& n0, int& k0) {
  int nb, kb;
  tile_coords_at(b, g.nbn, g.nbk, nb, kb);
  n0 = (g.nb_base + nb) * kRows;
  k0 = (g.kb_base + kb) * kCols;
}

// ---- launch plans (host)
// The region of a whole weight on the LDS-DMA paths: every 256-row and 128-column block.
inline GemmArgs whole_dma(const GemmArgs& g) {
  GemmArgs r = g;
  r.nb_base = 0;
  r.nbn = (int)(g.N / kRows);
  r.kb_base = 0;
  r.nbk = (int)(g.K / kCols);
  return r;
}

// 256 x 128 path with half tiles.  With F full tiles and S workgroup slots, the last round
// holds F mod S tiles and leaves CUs with one workgroup; turning the last c column blocks into
// 128 x 128 half tiles (c = the fewest columns that hold that remainder) ends the launch with a
// round of half tiles instead.  Sets nfull and kb_split; returns the grid size.
inline unsigned plan_split(GemmArgs& g, int slots) {
  const int nbN = g.nbn, nbK = g.nbk;
  const int full = nbN * nbK;
  const int rem = full % slots;
  const int c0 = rem == 0 ? 0 : (rem + nbN - 1) / nbN;
  const int c = c0 < nbK ? c0 : nbK;
  g.kb_split = nbK - c;
  g.nfull = nbN * g.kb_split;
  return (unsigned)(g.nfull + 2 * nbN * c);
}

// Wide 256 x 256 tiles in one workgroup of 8 waves per CU: a faster contraction than two
// 256 x 128 workgroups, but no other workgroup on the CU overlaps a tile's epilogue.  A wide
// launch should end in whole rounds.
//  * bf16 inputs, T >= 4096, every tile wide (K % 256 == 0) and R wide tiles leaving
//    R mod C = r over the C CUs: the last r / (N / 256) 256-column blocks (or the last
//    r / (K / 256) row blocks), whichever divides, become 2 r half-wide tiles of 128 x 256 in
//    the same launch.  Half of them go first, the rest after the wide tiles: the CUs that
//    start on a half-wide tile then run half a tile out of phase with the others, so the
//    epilogues' streams of W, m and v do not all fall in the same interval (at down_proj,
//    T = 4096: 567 us against 582 us with all half-wide tiles last, and 600 us on 256 x 128
//    tiles).
//  * Otherwise, for T >= 8192 (where the faster contraction outweighs the unoverlapped
//    epilogue; at T = 4096 the two tied): the first kw 256-column blocks of every row block,
//    kw the largest count for which N / 256 * kw is a positive multiple of the CU count, or,
//    where no column count works and K is a multiple of 256, the first nw row blocks over all
//    columns, nw the largest such count; the rest of the weight runs on the 256 x 128 path.
//    fp8 inputs only take this form.
constexpr int64_t kWideHalvesMinT = 4096, kWideMinT = 8192;
struct WidePlan {
  int kw = 0, nw = 0;  // whole rounds on part of the weight
  int hc = 0, hr = 0;  // bf16: the whole weight, the last hc column or hr row blocks half-wide
};

inline WidePlan plan_wide(const GemmArgs& g, int cus, bool halves) {
  WidePlan p;
  if (g.T < kWideHalvesMinT || cus <= 0) return p;
  const int nbN = (int)(g.N / kRows), nbK2 = (int)(g.K / (2 * kCols));
  if (halves && g.K % (2 * kCols) == 0 && nbN * nbK2 > cus) {
    const int r = (nbN * nbK2) % cus;
    if (r > 0 && r % nbN == 0) {
      p.hc = r / nbN;
      return p;
    }
    if (r > 0 && r % nbK2 == 0) {
      p.hr = r / nbK2;
      return p;
    }
  }
  if (g.T < kWideMinT) return p;
  for (int kw = nbK2; kw > 0; --kw)
    if ((nbN * kw) % cus == 0) {
      p.kw = kw;
      return p;
    }
  if (g.K % (2 * kCols) == 0)  // rows of wide tiles span every column
    for (int nw = nbN; nw > 0; --nw)
      if ((nw * nbK2) % cus == 0) {
        p.nw = nw;
        return p;
      }
  return p;
}

// The 256 x 128 path needs N % 256 == 0 and at least 128 of its tiles (256 workgroups once the
// plan turns them into half tiles); fp8 inputs at least 256 tiles.
inline bool use_v2(int in_type, const GemmArgs& g) {
  return in_type == FORGE_IN_BF16 && g.N % kRows == 0 && (g.N / kRows) * (g.K / kCols) >= 128;
}
inline bool use_v8(int in_type, const GemmArgs& g) {
  return in_type == FORGE_IN_FP8 && g.N % kRows == 0 && (g.N / kRows) * (g.K / kCols) >= 256;
}

// One kernel launch of a plan.
enum : int { LAUNCH_WIDE = 0, LAUNCH_V2 = 1, LAUNCH_V8 = 2, LAUNCH_SMALL = 3 };
struct Launch {
  int kind;
  GemmArgs g;
  unsigned grid;  // workgroups
  int tile;       // LAUNCH_SMALL: side of the square tiles (128 or 64)
};

// Register-staged path: fp32 inputs, whose MFMA rate is a sixteenth of bf16's, are bound by the
// matrix cores of the CUs that hold a tile; with fewer 128 x 128 tiles than CUs they take
// 64 x 64 tiles (four times the workgroups, each a quarter of the work).
inline int small_tile(int in_type, const GemmArgs& g, int cus) {
  const long tiles = (long)(g.N / kSmallTile) * (long)(g.K / kSmallTile);
  return in_type == FORGE_IN_F32 && tiles < cus ? 64 : kSmallTile;
}

// The launches of the fused step (fused = 1) or of the GEMM (fused = 0) for inputs of type
// in_type on a device with `cus` compute units (two workgroup slots each on the 256 x 128
// path): wide tiles first where they apply (fused step only), then the rest.  Returns the
// number of launches (0 to 2).
inline int plan_launches(int in_type, const GemmArgs& g, int cus, int fused, Launch (&out)[2]) {
  int n = 0;
  if (use_v2(in_type, g) || use_v8(in_type, g)) {
    const int kind = use_v2(in_type, g) ? LAUNCH_V2 : LAUNCH_V8;
    GemmArgs rest = whole_dma(g);
    const WidePlan wp = fused ? plan_wide(g, cus, kind == LAUNCH_V2) : WidePlan{};
    if (wp.hc > 0 || wp.hr > 0) {  // the whole weight in one launch with half-wide tiles
      GemmArgs w = rest;
      if (wp.hc > 0) {
        w.kb_split = w.nbk - 2 * wp.hc;
        w.h_nb = 0, w.hn = w.nbn, w.h_kb = w.kb_split, w.hk = 2 * wp.hc;
      } else {
        w.nbn -= wp.hr;
        w.kb_split = w.nbk;
        w.h_nb = w.nbn, w.hn = wp.hr, w.h_kb = 0, w.hk = w.nbk;
      }
      w.nfull = w.nbn * (w.kb_split / 2);
      const int nhalf = w.hn * w.hk;
      w.nfront = (nhalf / 2) & ~7;
      out[n++] = Launch{LAUNCH_WIDE, w, (unsigned)(w.nfull + nhalf), 0};
      return n;
    }
    if (wp.kw > 0 || wp.nw > 0) {
      GemmArgs wide = rest;
      if (wp.kw > 0) {
        wide.nbk = 2 * wp.kw;
        rest.kb_base = 2 * wp.kw;
        rest.nbk -= 2 * wp.kw;
      } else {
        wide.nbn = wp.nw;
        rest.nb_base = wp.nw;
        rest.nbn -= wp.nw;
      }
      wide.kb_split = wide.nbk;
      wide.nfull = wide.nbn * (wide.nbk / 2);
      out[n++] = Launch{LAUNCH_WIDE, wide, (unsigned)wide.nfull, 0};
      if (rest.nbn == 0 || rest.nbk == 0) return n;
    }
    const unsigned grid = kind == LAUNCH_V2 ? plan_split(rest, 2 * cus) : (unsigned)(rest.nbn * rest.nbk);
    out[n++] = Launch{kind, rest, grid, 0};
    return n;
  }
  const int t = small_tile(in_type, g, cus);
  out[n++] = Launch{LAUNCH_SMALL, g, (unsigned)((g.N / t) * (g.K / t)), t};
  return n;
}

// ---- work queues of the one-launch backward step (forge_backward.hip)
// Three phases of work items, in order: 0 the dX tiles, 1 the step's full tiles, 2 its half
// tiles.  Each phase is spread over 8 queues, one per XCD slot: the k-th claim on queue q of a
// phase returns its item q + 8 k while k < queue_size(n, q), so the items a queue hands out are
// those the separate launches give workgroups q, q + 8, q + 16, ... of the XCD q.
constexpr int kQueues = 8, kPhases = 3;

struct BackwardItems {
  int dgrad, full, half;  // items per phase
};
__host__ __device__ inline BackwardItems backward_items(const GemmArgs& g, int nbT) {
  return BackwardItems{nbT * g.nbk, g.nfull, 2 * g.nbn * (g.nbk - g.kb_split)};
}
__host__ __device__ inline int phase_items(const BackwardItems& it, int p) {
  return p == 0 ? it.dgrad : p == 1 ? it.full : it.half;
}
__host__ __device__ inline int queue_size(int n, int q) { return n / kQueues + (q < n % kQueues ? 1 : 0); }

// The queue a workgroup of XCD slot q0 claims from, given which queues were open (bit 8 p + q of
// `open` set: claims on queue q of phase p had not yet used up its items) in one snapshot of the
// claim counters: the earliest phase with an open queue, and in it queue q0 or the next open one
// after it.  False if no queue was open.
__host__ __device__ inline bool pick_queue(uint32_t open, int q0, int& phase, int& queue) {
  if (open == 0) return false;
  phase = __builtin_ctz(open) / kQueues;
  const uint32_t pm = (open >> (kQueues * phase)) & 0xFFu;
  const uint32_t rot = ((pm >> q0) | (pm << (kQueues - q0))) & 0xFFu;
  queue = (q0 + __builtin_ctz(rot)) & (kQueues - 1);
  return true;
}

// The item the k-th claim on queue q of a phase of n items returns, or -1 once the queue's items
// are used up.
__host__ __device__ inline int claimed_item(int n, int q, int k) {
  return k < queue_size(n, q) ? q + kQueues * k : -1;
}

}  // namespace plan
}  // namespace forge
