// forge_fused8.h -- the fused step for fp8 e4m3 inputs on the LDS-DMA path with 8-bit
// transpose reads (forge_mainloop8.h): 256 x 128 tiles, and 256 x 256 tiles in one 8-wave
// workgroup per CU for long token counts.  FORGE explainer (gist.science), Technical Summary
// section 2 "Core Mechanism" and section 4 (fp8 composability).
//
// Instantiated per moment format in forge_fused8_f32.hip, forge_fused8_q8.hip (linear 8-bit
// map) and forge_fused8_q8d.hip (dynamic 8-bit map).
#pragma once

#include "forge_epilogue.h"

namespace forge {

// fp8 e4m3 inputs, 256 x 128 tiles fed by LDS DMA with 8-bit transpose reads
// (forge_mainloop8.h); the tensors' scale product multiplies the finished sums at staging.
static_assert(ml8::SMEM <= kSmem2, "fp8 stages fit the shared buffer size");

// The launch covers the nbn 256-row blocks from nb_base on and the nbk 128-column blocks from
// kb_base on.
template <int WT, int ST, int OPT>
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void fused_step_kernel8(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  int n0, k0;
  plan::tile8(g, (int)blockIdx.x, n0, k0);
  ml8::floatx16 acc[4][2];
  ml8::contract(acc, smem, g, n0, k0);
  const float scale = g.dy_scale[0] * g.x_scale[0];
  float* st = reinterpret_cast<float*>(smem);
  tile_epilogue<OPT, WT, ST, 2, false>(g, e, smem, n0, k0, [&](int h) { ml8::stage_acc_half(st, acc, scale, h); });
}

// fp8 e4m3 inputs on 256 x 256 tiles, one workgroup of 8 waves per CU (forge_mainloop8.h, wide
// tiles); each 128-column half runs the epilogue from its own staging buffer.
constexpr int kSmem8W = ml8::W_SMEM > 2 * ml2::EPI_BYTES ? ml8::W_SMEM : 2 * ml2::EPI_BYTES;
static_assert(kSmem8W <= 160 * 1024, "wide fp8 tiles fit the CU's LDS");

template <int WT, int ST, int OPT>
__global__ __launch_bounds__(2 * ml2::THREADS, 1) void fused_step_kernel8w(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem8W];
  int n0, kw0;
  plan::wide_tile(g, (int)blockIdx.x, n0, kw0);
  const int kh = (int)(threadIdx.x >> 8);
  ml8::floatx16 acc[4][2];
  ml8::contract_wide(acc, smem, g, n0, kw0);
  const float scale = g.dy_scale[0] * g.x_scale[0];
  unsigned char* mine = smem + kh * ml2::EPI_BYTES;
  float* st = reinterpret_cast<float*>(mine);
  tile_epilogue<OPT, WT, ST, 2, false>(g, e, mine, n0, kw0 + kh * ml2::BN,
                                       [&](int h) { ml8::stage_acc_half(st, acc, scale, h); });
}

template <int ST>
FusedFn select_fused8(int wide, int w_type, int opt) {
  if (w_type == FORGE_W_BF16) {
    switch (opt) {
#define FORGE_CASE(O) \
  case O: return wide ? fused_step_kernel8w<FORGE_W_BF16, ST, O> : fused_step_kernel8<FORGE_W_BF16, ST, O>;
      FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
    }
  } else {
    switch (opt) {
#define FORGE_CASE(O) \
  case O: return wide ? fused_step_kernel8w<FORGE_W_F32, ST, O> : fused_step_kernel8<FORGE_W_F32, ST, O>;
      FORGE_FOR_EACH_OPT(FORGE_CASE)
#undef FORGE_CASE
    }
  }
  return nullptr;
}

}  // namespace forge
