// forge_fused2.h -- the fused step for bf16 inputs on the LDS-DMA path (forge_mainloop2.h):
// 256 x 128 tiles, two workgroups per CU, with 128 x 128 half tiles balancing the last round of
// a launch, and 256 x 256 tiles in one 8-wave workgroup per CU, with 128 x 256 half-wide tiles
// balancing theirs (the launch plans are in forge_plan.h).
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism".
//
// Instantiated per moment format in forge_fused2_f32.hip, forge_fused2_q8.hip (linear 8-bit
// map) and forge_fused2_q8d.hip (dynamic 8-bit map).
#pragma once

#include "forge_epilogue.h"

namespace forge {

static_assert(ml2::BM == plan::kRows && ml2::BN == plan::kCols && ml2::BM_HALF == plan::kHalfRows,
              "the launch plans and the kernels use the same tiles");

// Full 256 x 128 tile at (n0, k0): contraction, then the epilogue over its two 128-row halves.
// before_update() runs between the two (the one-launch backward step waits there until no
// dgrad tile still reads this tile's old weight).
template <int WT, int ST, int OPT, class BeforeUpdate>
__device__ __forceinline__ void fused_full_tile_at(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                                   int k0, BeforeUpdate&& before_update) {
  ml2::floatx4 acc[8][4];
  ml2::contract<Pipe2>(acc, smem, g, n0, k0);
  if (!before_update()) return;
  float* st = reinterpret_cast<float*>(smem);
  tile_epilogue<OPT, WT, ST, 2, true>(g, e, smem, n0, k0, [&](int h) { ml2::stage_acc_half(st, acc, 1.0f, h); });
}

// Half 128 x 128 tile at (n0, k0): all 128 rows staged at once.
template <int WT, int ST, int OPT, class BeforeUpdate>
__device__ __forceinline__ void fused_half_tile_at(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                                   int k0, BeforeUpdate&& before_update) {
  ml2::floatx4 acc[4][4];
  ml2::contract<Pipe2H>(acc, smem, g, n0, k0);
  if (!before_update()) return;
  float* st = reinterpret_cast<float*>(smem);
  tile_epilogue<OPT, WT, ST, 1, true>(g, e, smem, n0, k0, [&](int) { ml2::stage_acc_all(st, acc, 1.0f); });
}

// Full tile b of the launch's full tiles [0, nfull), and half tile hb of the blocks
// [kb_split, nbk).
template <int WT, int ST, int OPT>
__device__ __forceinline__ void fused_full_tile(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int b) {
  int n0, k0;
  plan::full_tile(g, b, n0, k0);
  fused_full_tile_at<WT, ST, OPT>(g, e, smem, n0, k0, [] { return true; });
}
template <int WT, int ST, int OPT>
__device__ __forceinline__ void fused_half_tile(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int hb) {
  int n0, k0;
  plan::half_tile(g, hb, n0, k0);
  fused_half_tile_at<WT, ST, OPT>(g, e, smem, n0, k0, [] { return true; });
}

template <int WT, int ST, int OPT>
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void fused_step_kernel2(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  const int b = (int)blockIdx.x;
  if (b < g.nfull) fused_full_tile<WT, ST, OPT>(g, e, smem, b);
  else fused_half_tile<WT, ST, OPT>(g, e, smem, b - g.nfull);
}

// bf16 inputs, 256 x 256 tiles, one workgroup of 8 waves per CU (forge_mainloop2.h, wide
// tiles): both 128-column halves share the dY panel and 4 slabs fit in LDS.  The epilogue is
// the 256 x 128 tile's, run by each half: threads 0-255 update columns k0 .. k0 + 127 and
// threads 256-511 columns k0 + 128 .. k0 + 255, each staging through its own LDS buffer.  A
// launch may also hold 128 x 256 half-wide tiles, whose halves run the 128 x 128 tile's
// epilogue (plan::wide_item gives each workgroup its tile).
constexpr int kSmemW = ml2::WidePipe::SMEM > 2 * ml2::EPI_BYTES ? ml2::WidePipe::SMEM : 2 * ml2::EPI_BYTES;
static_assert(kSmemW <= 160 * 1024 && ml2::WideHalfPipe::SMEM <= kSmemW, "wide tiles fit the CU's LDS");

template <int WT, int ST, int OPT>
__global__ __launch_bounds__(2 * ml2::THREADS, 1) void fused_step_kernel2w(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemW];
  int n0, kw0;
  const bool half = plan::wide_item(g, (int)blockIdx.x, n0, kw0);
  const int kh = (int)(threadIdx.x >> 8);
  unsigned char* mine = smem + kh * ml2::EPI_BYTES;
  float* st = reinterpret_cast<float*>(mine);
  if (half) {
    ml2::floatx4 acc[4][4];
    ml2::contract_wide<ml2::WideHalfPipe>(acc, smem, g, n0, kw0);
    tile_epilogue<OPT, WT, ST, 1, true>(g, e, mine, n0, kw0 + kh * ml2::BN,
                                        [&](int) { ml2::stage_acc_all(st, acc, 1.0f); });
  } else {
    ml2::floatx4 acc[8][4];
    ml2::contract_wide<ml2::WidePipe>(acc, smem, g, n0, kw0);
    tile_epilogue<OPT, WT, ST, 2, true>(g, e, mine, n0, kw0 + kh * ml2::BN,
                                        [&](int h) { ml2::stage_acc_half(st, acc, 1.0f, h); });
  }
}

template <int ST>
FusedFn select_fused2(int wide, int w_type, int opt) {
  if (w_type == FORGE_W_BF16) {
    switch (opt) {
#define FORGE_CASE(O) \
  case O: return wide ? fused_step_kernel2w<FORGE_W_BF16, ST, O> : fused_step_kernel2<FORGE_W_BF16, ST, O>;
      FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
    }
  } else {
    switch (opt) {
#define FORGE_CASE(O) \
  case O: return wide ? fused_step_kernel2w<FORGE_W_F32, ST, O> : fused_step_kernel2<FORGE_W_F32, ST, O>;
      FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
    }
  }
  return nullptr;
}

}  // namespace forge
