// forge_fused1.h -- the fused step on 128 x 128 (or, for small fp32 layers, 64 x 64) tiles with
// register-staged operands (forge_mainloop.h): fp32 inputs, and bf16 / fp8 layers too small for
// the LDS-DMA paths.
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism".
//
// Instantiated per input format in forge_fused1_f32.hip, forge_fused1_bf16.hip and
// forge_fused1_fp8.hip.
#pragma once

#include "forge_epilogue.h"

namespace forge {

template <int IN, int WT, int ST, int OPT, int S>
__global__ __launch_bounds__(kThreads, S == 128 ? 2 : 4) void fused_step_kernel(GemmArgs g, EpiArgs e) {
  using TL = SmallTile<S>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[TL::SMEM];
  const int nbN = (int)(g.N / S), nbK = (int)(g.K / S);
  int nb, kb;
  tile_coords(nbN, nbK, nb, kb);
  const int n0 = nb * S, k0 = kb * S;

  floatx4 acc[TL::NB][TL::NB];
  contract_tile<IN, S>(acc, smem, g, n0, k0);

  // the thread's segments of 16 elements (4 for S = 128, 1 for S = 64); the next segment's
  // stored state is in flight while one is updated, and the first leaves before the staging
  auto index_of = [&](int s) {
    int row, col;
    small_seg<S>(s, row, col);
    return (uint32_t)(n0 + row) * (uint32_t)g.K + (uint32_t)(k0 + col);
  };
  SegIn xs[2];
  seg_load<OPT, WT, ST>(xs[0], index_of(0), e);
  float* st = reinterpret_cast<float*>(smem);
  stage_acc<S>(st, acc, input_scale<IN>(g));
  __syncthreads();
  static_for<TL::SEGS>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    if constexpr (s + 1 < TL::SEGS) seg_load<OPT, WT, ST>(xs[(s + 1) & 1], index_of(s + 1), e);
    int row, col;
    small_seg<S>(s, row, col);
    float gr[16];
    read_seg16(gr, st, row, col);
    seg_apply<OPT, WT, ST>(gr, index_of(s), xs[s & 1], e);
  });
}

// tile = 64 selects the 64 x 64 tiles, which only fp32 inputs have (the launch plan asks for
// them for fp32 layers with fewer 128 x 128 tiles than CUs); 128 otherwise.
template <int IN, int S>
FusedFn select_fused1_tile(int w_type, int s_type, int opt) {
  switch (opt) {
#define FORGE_CASE(O)                                                                                       \
  case O:                                                                                                   \
    if (w_type == FORGE_W_BF16)                                                                             \
      return s_type == FORGE_S_F32  ? fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_F32, O, S>                 \
             : s_type == FORGE_S_Q8 ? fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_Q8, O, S>                  \
                                    : fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_Q8D, O, S>;                \
    return s_type == FORGE_S_F32  ? fused_step_kernel<IN, FORGE_W_F32, FORGE_S_F32, O, S>                    \
           : s_type == FORGE_S_Q8 ? fused_step_kernel<IN, FORGE_W_F32, FORGE_S_Q8, O, S>                     \
                                  : fused_step_kernel<IN, FORGE_W_F32, FORGE_S_Q8D, O, S>;
    FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
  }
  return nullptr;
}

template <int IN>
FusedFn select_fused1(int w_type, int s_type, int opt, int tile) {
  if constexpr (IN == FORGE_IN_F32)
    if (tile == 64) return select_fused1_tile<IN, 64>(w_type, s_type, opt);
  return tile == 128 ? select_fused1_tile<IN, 128>(w_type, s_type, opt) : nullptr;
}

}  // namespace forge
