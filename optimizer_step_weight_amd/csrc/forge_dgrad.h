// forge_dgrad.h -- dX = dY W tiles on the LDS-DMA path (bf16 in, fp32 accumulate, bf16
// nearest-even out), shared by the dgrad kernels and the one-launch backward step.
// FORGE explainer (gist.science), Technical Summary section 5, limitations: the input gradient
// is computed from the weight as it was before the update.
#pragma once

#include "forge_epilogue.h"

namespace forge {

// dX rows t0 .. t0 + 127 of the staged rows of one 128-column block at k0, as bf16 (rows at or
// past T are not written).
__device__ __forceinline__ void store_dx_rows(const float* st, uint16_t* dX, int64_t T, int64_t K, int64_t t0,
                                              int k0) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int row, kseg;
    seg_pos(s, row, kseg);
    const int64_t t = t0 + row;
    if (t >= T) continue;
    float gr[16];
    staged_grad(st, s, gr);
    u32x4 a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = f32_to_bf16_rne(gr[2 * q]) | (f32_to_bf16_rne(gr[2 * q + 1]) << 16);
      b[q] = f32_to_bf16_rne(gr[8 + 2 * q]) | (f32_to_bf16_rne(gr[8 + 2 * q + 1]) << 16);
    }
    uint16_t* d = dX + t * K + k0 + kseg * 16;
    st16(d, a);
    st16(d + 8, b);
  }
}

// The 256-token x 128-column dX tile at (t0, k0), one workgroup of 4 waves; the reduction over N
// in 32-wide slabs (forge_mainloop2.h, dgrad section).  contracted() runs once, after the
// contraction's final barrier: by then every read of W for this tile has completed.
template <class Contracted>
__device__ __forceinline__ void dgrad_tile(const uint16_t* dY, const uint16_t* W, uint16_t* dX, int64_t T, int64_t N,
                                           int64_t K, int64_t t0, int k0, unsigned char* smem,
                                           Contracted&& contracted) {
  ml2::floatx4 acc[8][4];
  ml2::dgrad_contract(acc, smem, dY, W, T, N, K, t0, k0);
  contracted();
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    ml2::stage_acc_half(st, acc, 1.0f, half);
    __syncthreads();
    store_dx_rows(st, dX, T, K, t0 + half * ml2::EPI_ROWS, k0);
    __syncthreads();
  }
}

// The 256-token x 256-column dX tile at (t0, k0), one workgroup of 8 waves (forge_mainloop2.h,
// wide dgrad tiles): both 128-column halves share the dY slab; each stages its accumulators
// through its own LDS buffer.
__device__ __forceinline__ void dgrad_tile_wide(const uint16_t* dY, const uint16_t* W, uint16_t* dX, int64_t T,
                                                int64_t N, int64_t K, int64_t t0, int k0, unsigned char* smem) {
  const int kh = (int)(threadIdx.x >> 8);
  ml2::floatx4 acc[8][4];
  ml2::dgrad_wide_contract(acc, smem, dY, W, T, N, K, t0, k0);
  float* st = reinterpret_cast<float*>(smem + kh * ml2::EPI_BYTES);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    ml2::stage_acc_half(st, acc, 1.0f, half);
    __syncthreads();
    store_dx_rows(st, dX, T, K, t0 + half * ml2::EPI_ROWS, k0 + kh * ml2::BN);
    __syncthreads();
  }
}

}  // namespace forge
