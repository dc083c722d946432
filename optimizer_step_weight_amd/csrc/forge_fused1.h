// forge_fused1.h -- the fused step on 128 x 128 tiles with register-staged operands
// (forge_mainloop.h): fp32 inputs, and bf16 / fp8 layers too small for the LDS-DMA paths.
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism".
//
// Instantiated per input format in forge_fused1_f32.hip, forge_fused1_bf16.hip and
// forge_fused1_fp8.hip.
#pragma once

#include "forge_epilogue.h"

namespace forge {

template <int IN, int WT, int ST, int OPT>
__global__ __launch_bounds__(kThreads, 2) void fused_step_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  const int nbN = (int)(g.N / kBM), nbK = (int)(g.K / kBN);
  int nb, kb;
  tile_coords(nbN, nbK, nb, kb);
  const int n0 = nb * kBM, k0 = kb * kBN;

  floatx4 acc[4][4];
  contract_tile<IN>(acc, smem, g, n0, k0);

  // the thread's 4 segments of 16 elements; the next segment's stored state is in flight while
  // one is updated, and the first leaves before the staging
  const int tid = threadIdx.x;
  auto index_of = [&](int s) {
    const int seg = tid + kThreads * s, row = seg >> 3, kseg = seg & 7;
    return (uint32_t)(n0 + row) * (uint32_t)g.K + (uint32_t)(k0 + kseg * 16);
  };
  SegIn xs[2];
  seg_load<OPT, WT, ST>(xs[0], index_of(0), e);
  float* st = reinterpret_cast<float*>(smem);
  stage_acc(st, acc, input_scale<IN>(g));
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) seg_load<OPT, WT, ST>(xs[(s + 1) & 1], index_of(s + 1), e);
    const int seg = tid + kThreads * s, row = seg >> 3, kseg = seg & 7;
    float gr[16];
    read_seg16(gr, st, row, kseg);
    seg_apply<OPT, WT, ST>(gr, index_of(s), xs[s & 1], e);
  }
}

template <int IN>
FusedFn select_fused1(int w_type, int s_type, int opt) {
  switch (opt) {
#define FORGE_CASE(O)                                                                                       \
  case O:                                                                                                   \
    if (w_type == FORGE_W_BF16)                                                                             \
      return s_type == FORGE_S_F32  ? fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_F32, O>                    \
             : s_type == FORGE_S_Q8 ? fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_Q8, O>                     \
                                    : fused_step_kernel<IN, FORGE_W_BF16, FORGE_S_Q8D, O>;                   \
    return s_type == FORGE_S_F32  ? fused_step_kernel<IN, FORGE_W_F32, FORGE_S_F32, O>                       \
           : s_type == FORGE_S_Q8 ? fused_step_kernel<IN, FORGE_W_F32, FORGE_S_Q8, O>                        \
                                  : fused_step_kernel<IN, FORGE_W_F32, FORGE_S_Q8D, O>;
    FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
  }
  return nullptr;
}

}  // namespace forge
