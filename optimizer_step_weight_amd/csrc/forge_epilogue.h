// forge_epilogue.h -- the optimizer epilogue of a contracted tile, shared by the fused kernels
// and the unfused optimizer kernel.
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": once a tile's
// gradient is complete in fp32 registers, the element-wise rule is applied to it and only the
// weight and its moments are written back.  The gradient passes through the workgroup's LDS to
// be re-laid out for vector memory access (16 consecutive columns per thread, or 4-element
// units with consecutive lanes on consecutive units); it never reaches HBM.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "forge_mainloop.h"
#include "forge_mainloop2.h"
#include "forge_mainloop8.h"
#include "forge_paths.h"

namespace forge {

template <int IN>
__device__ __forceinline__ float input_scale(const GemmArgs& g) {
  if constexpr (IN == FORGE_IN_FP8) return g.dy_scale[0] * g.x_scale[0];
  return 1.0f;
}

// bf16 inputs, 256 x 128 workgroup tiles fed by LDS DMA (forge_mainloop2.h): 32-token slabs,
// three in LDS (72 KiB), so two workgroups share a CU and each SIMD runs two waves.  The
// launcher may turn the last k-block columns into 128 x 128 half tiles (four 32-token slabs in
// LDS) so that the last round of workgroups fills the chip (plan::plan_split, forge_plan.h).
using Pipe2 = ml2::Pipe<32, 3>;
using Pipe2H = ml2::Pipe<32, 4, 4>;
constexpr int kOcc2 = 2;
constexpr int kSmem2 = Pipe2::SMEM;
static_assert(Pipe2H::SMEM <= kSmem2 && ml2::EPI_BYTES <= kSmem2, "half tiles and the staging share the LDS");

// Epilogue helpers index threads within a group of 256 (a whole 256-thread workgroup, or one
// 128-column half of an 8-wave workgroup).
__device__ __forceinline__ int group_tid() { return (int)(threadIdx.x & (ml2::THREADS - 1)); }

// The thread's 16-element segment s (0..3) of 128 staged rows: row and column in the staging.
__device__ __forceinline__ void seg_pos(int s, int& row, int& kseg) {
  const int seg = group_tid() + ml2::THREADS * s;
  row = seg >> 3;
  kseg = seg & 7;
}

__device__ __forceinline__ void staged_grad(const float* st, int s, float (&gr)[16]) {
  int row, kseg;
  seg_pos(s, row, kseg);
  const float* p = st + row * ml2::EPI_LD + kseg * 16;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(p + 4 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) gr[4 * q + c] = x[c];
  }
}

// ---- epilogue in the lane-contiguous unit layout (forge_device.h, "one 4-element unit")
// 128 staged rows are 16 rounds of 8 rows: in round rho this thread's unit is row
// 8 rho + 2 wave + lane / 32, columns 4 (lane % 32) .. +3, so a wave touches two contiguous row
// segments per access.  Batches of 4 rounds share one Philox block per quad.
__device__ __forceinline__ int unit_row(int rho) {
  return 8 * rho + 2 * (group_tid() >> 6) + ((group_tid() & 63) >> 5);
}
__device__ __forceinline__ int unit_col() { return 4 * (int)(threadIdx.x & 31); }

// rows0: the tile row of staged row 0 (n0 + 128 half)
__device__ __forceinline__ uint32_t unit_index(const GemmArgs& g, int rows0, int k0, int rho) {
  return (uint32_t)(rows0 + unit_row(rho)) * (uint32_t)g.K + (uint32_t)(k0 + unit_col());
}

template <int OPT, int WT, int ST>
__device__ __forceinline__ void unit_batch_load(UnitIn (&x)[4], const GemmArgs& g, const EpiArgs& e, int rows0,
                                                int k0, int batch) {
#pragma unroll
  for (int r = 0; r < 4; ++r) unit_load<OPT, WT, ST>(x[r], unit_index(g, rows0, k0, 4 * batch + r), e);
}

// The stochastic-rounding words of a batch (zero when they are not used).
template <int WT>
__device__ __forceinline__ void unit_batch_words(uint64_t (&w)[4], const GemmArgs& g, const EpiArgs& e, int rows0,
                                                 int k0, int batch) {
#pragma unroll
  for (int r = 0; r < 4; ++r) w[r] = 0ull;
  if (WT == FORGE_W_BF16 && e.sr) {
    uint32_t i[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) i[r] = unit_index(g, rows0, k0, 4 * batch + r);
    sr_words4(i, e, w);
  }
}

template <int OPT, int WT, int ST>
__device__ __forceinline__ void unit_batch_apply(const UnitIn (&x)[4], const uint64_t (&w)[4], const float* st,
                                                 const GemmArgs& g, const EpiArgs& e, int rows0, int k0, int batch) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const floatx4 q = *reinterpret_cast<const floatx4*>(st + unit_row(4 * batch + r) * ml2::EPI_LD + unit_col());
    const float gr[4] = {q[0], q[1], q[2], q[3]};
    unit_apply<OPT, WT, ST>(gr, unit_index(g, rows0, k0, 4 * batch + r), x[r], w[r], e);
  }
}

// The whole epilogue of a tile of HALVES x 128 rows: stage(h) writes rows [128 h, 128 h + 128)
// into the staging.  The next batch's stored state is in flight while one is updated; the
// first batch's loads leave before the first staging.
template <int OPT, int WT, int ST, int HALVES, class Stage>
__device__ __forceinline__ void unit_epilogue(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                              int k0, Stage&& stage) {
  float* st = reinterpret_cast<float*>(smem);
  UnitIn xa[4], xb[4];
  // one batch: words, the next batch's loads, then this batch's updates
  auto batch = [&](UnitIn (&cur)[4], UnitIn (&nxt)[4], int h, int b) {
    const int rows0 = n0 + 128 * h;
    uint64_t w[4];
    unit_batch_words<WT>(w, g, e, rows0, k0, b);
    if (b < 3) unit_batch_load<OPT, WT, ST>(nxt, g, e, rows0, k0, b + 1);
    else if (h + 1 < HALVES) unit_batch_load<OPT, WT, ST>(nxt, g, e, rows0 + 128, k0, 0);
    unit_batch_apply<OPT, WT, ST>(cur, w, st, g, e, rows0, k0, b);
  };
  unit_batch_load<OPT, WT, ST>(xa, g, e, n0, k0, 0);
  static_for<HALVES>([&](auto hc) {  // the staging of half h reads accumulators chosen by h
    constexpr int h = decltype(hc)::value;
    stage(h);
    __syncthreads();
    batch(xa, xb, h, 0);
    batch(xb, xa, h, 1);
    batch(xa, xb, h, 2);
    batch(xb, xa, h, 3);
    __syncthreads();
  });
}

// Segment epilogue: 16 consecutive elements of a row per thread (4 per 128-row half).  Used
// for int8 moments: with 1-byte codes and per-block scales the 4-element units take about 3x
// more small memory instructions per element than 16-element segments, and the
// contiguous-lane layout gains little on such narrow data.  With bf16 weights the next
// segment's stored state (18 registers with int8 moments) is loaded before the current one is
// updated, so its latency hides behind that update.  fp32 weights and Lion keep one segment
// in flight (loaded after the update), which their registers allow without spilling.  The
// first segment's loads leave before the staging.
template <int OPT, int WT, int ST>
constexpr bool seg_ahead() {
  return WT == FORGE_W_BF16 && OPT != FORGE_OPT_LION;
}

template <int OPT, int WT, int ST, int HALVES, class Stage>
__device__ __forceinline__ void seg_epilogue(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                             int k0, Stage&& stage) {
  float* st = reinterpret_cast<float*>(smem);
  auto index_of = [&](int j) {  // the thread's j-th segment (j = 4 half + s)
    int row, kseg;
    seg_pos(j & 3, row, kseg);
    return (uint32_t)(n0 + (j >> 2) * ml2::EPI_ROWS + row) * (uint32_t)g.K + (uint32_t)(k0 + kseg * 16);
  };
  constexpr bool AHEAD = seg_ahead<OPT, WT, ST>();
  SegIn xs[AHEAD ? 2 : 1];
  seg_load<OPT, WT, ST>(xs[0], index_of(0), e);
  static_for<HALVES>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    stage(h);
    __syncthreads();
    static_for<4>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int j = 4 * h + s;
      constexpr bool more = j + 1 < 4 * HALVES;
      float gr[16];
      if constexpr (AHEAD) {
        if (more) seg_load<OPT, WT, ST>(xs[(j + 1) & 1], index_of(j + 1), e);
        staged_grad(st, s, gr);
        seg_apply<OPT, WT, ST>(gr, index_of(j), xs[j & 1], e);
      } else {
        staged_grad(st, s, gr);
        seg_apply<OPT, WT, ST>(gr, index_of(j), xs[0], e);
        if (more) seg_load<OPT, WT, ST>(xs[0], index_of(j + 1), e);
      }
    });
    __syncthreads();
  });
}

// The epilogue for the state format: 4-element units for fp32 moments, segments for int8
// (SEG_INT8; the fp8 kernel keeps units for int8, where the segment form does not fit its
// registers).
template <int OPT, int WT, int ST, int HALVES, bool SEG_INT8, class Stage>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                              int k0, Stage&& stage) {
  if constexpr (ST != FORGE_S_F32 && SEG_INT8) seg_epilogue<OPT, WT, ST, HALVES>(g, e, smem, n0, k0, stage);
  else unit_epilogue<OPT, WT, ST, HALVES>(g, e, smem, n0, k0, stage);
}

// dW rows of 128 staged rows, written with 16-byte stores.
__device__ __forceinline__ void store_staged(const float* st, float* dW, int64_t K, int n0, int k0) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int row, kseg;
    seg_pos(s, row, kseg);
    const float* p = st + row * ml2::EPI_LD + kseg * 16;
    float* d = dW + (int64_t)(n0 + row) * K + k0 + kseg * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(d + 4 * q, *reinterpret_cast<const u32x4*>(p + 4 * q));
  }
}

}  // namespace forge
