// forge_mainloop8.h -- token contraction of a 256 x 128 weight tile for fp8 e4m3 inputs with
// per-tensor scales, fed by global->LDS DMA and 8-bit LDS transpose reads.
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": the tile's
// gradient is accumulated over all tokens in fp32 registers; any order of the tokens is a
// valid summation order (section 2 "Precision and Fidelity").  The fp8 codes are multiplied
// as they are; the product of the two tensors' scales is applied once, to the finished sum,
// when the accumulators are staged for the epilogue.
//
// Data path (gfx950):
//  * A slab of 64 tokens of dY[:, n0:n0+256] (16 KiB, 256-byte token rows) and X[:, k0:k0+128]
//    (8 KiB, 128-byte rows) is copied to LDS by buffer_load_dwordx4 ... lds (16 bytes a lane,
//    1 KiB a wave, in lane order), three slabs in flight; tokens past T read as zero.
//  * v_mfma_scale_f32_32x32x64_f8f6f4 (both operands e4m3, unit block scales) consumes one
//    slab per k-step: lane l holds 32 codes of row / column l % 32, tokens 32 (l / 32) ..
//    +31.  ds_read_b64_tr_b8 builds them from token-major rows: within a 16-lane group, lane
//    j receives byte (j % 8) of the 8-byte pieces addressed by lanes 2 f + j / 8 (f = 0..7).
//    Lane i therefore points at token row (base + i / 2), columns c0 + 8 (i % 2) .. +7, and
//    lane j gets tokens base .. base + 7 of column c0 + j; four reads (base + 0, 8, 16, 24)
//    fill a fragment.
//  * Within one read the 32 lanes of a half wave touch 8 token rows x 32 bytes.  16-byte
//    chunks are XOR-swizzled so those land in distinct banks: chunk ^ 2 (t mod 8) in the
//    256-byte dY rows (one row spans all 64 banks), chunk ^ 2 ((t / 2) mod 4) in the
//    128-byte X rows (two rows share the 64 banks).
//
// Workgroup: 256 threads = 4 waves as 2 (n) x 2 (k); a wave holds 4 x 2 MFMA 32 x 32 blocks
// (16 accumulators each, 128 registers per lane) of 64 columns and 128 rows, two 32-row blocks
// in each 128-row half of the tile (as on the bf16 path), two workgroups per CU.
#pragma once

#include "forge_mainloop2.h"

namespace forge {
namespace ml8 {

using ml2::barrier;
using ml2::dma16;
using ml2::make_rsrc;
using ml2::wait_vm;
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int v2i32 __attribute__((ext_vector_type(2)));

constexpr int TK = 64, STAGES = 3;
constexpr int ROW_A = 256, ROW_B = 128;                 // bytes per token row (fp8 codes)
constexpr int PANEL_A = TK * ROW_A, PANEL_B = TK * ROW_B;  // 16 KiB, 8 KiB
constexpr int STAGE = PANEL_A + PANEL_B, SMEM = STAGES * STAGE;
constexpr int DMA_A = PANEL_A / 1024 / 4, DMA_B = PANEL_B / 1024 / 4, DMA = DMA_A + DMA_B;  // 4 + 2 per wave

__device__ __forceinline__ int swz_a(int row) { return 2 * (row & 7); }
__device__ __forceinline__ int swz_b(int row) { return 2 * ((row >> 1) & 3); }

struct Feed {
  u32x4 rA, rB;
  uint32_t offA[DMA_A], offB[DMA_B];
  uint32_t stepA, stepB;
};

// A 1 KiB DMA covers 4 dY rows (16 chunks each) or 8 X rows (8 chunks each).
__device__ __forceinline__ void make_feed(Feed& f, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                                          int n0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(dY, (uint32_t)(T * N));
  f.rB = make_rsrc(X, (uint32_t)(T * K));
#pragma unroll
  for (int j = 0; j < DMA_A; ++j) {
    const int d = DMA_A * wave + j, r = 4 * d + (lane >> 4), p = lane & 15;
    f.offA[j] = (uint32_t)(r * N + n0 + 16 * (p ^ swz_a(r)));
  }
#pragma unroll
  for (int j = 0; j < DMA_B; ++j) {
    const int x = DMA_B * wave + j, r = 8 * x + (lane >> 3), p = lane & 7;
    f.offB[j] = (uint32_t)(r * K + k0 + 16 * (p ^ swz_b(r)));
  }
  f.stepA = (uint32_t)(TK * N);
  f.stepB = (uint32_t)(TK * K);
}

__device__ __forceinline__ void issue(const Feed& f, unsigned char* stage, int slab) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < DMA_A; ++j) dma16(f.rA, f.offA[j] + sa, stage + (DMA_A * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < DMA_B; ++j) dma16(f.rB, f.offB[j] + sb, stage + PANEL_A + (DMA_B * wave + j) * 1024);
}

// 32 codes of column c0 + (lane % 32), tokens 32 (lane / 32) .. +31 of the slab: four
// transpose reads.  Lane i of a 16-lane group addresses token row base + i / 2 and the 8
// columns c0 + 16 g + 8 (i % 2) .. where g = (lane / 16) % 2 selects the column half.
// WIDE: 256-byte rows with the dY swizzle (the X panel of a wide tile).
template <bool IS_A, bool WIDE = false>
__device__ __forceinline__ intx8 frag(const unsigned char* panel, int c0) {
  constexpr bool A_LIKE = IS_A || WIDE;
  const int lane = threadIdx.x & 63, i = lane & 15, g = (lane >> 4) & 1, h = lane >> 5;
  const int col = c0 + 16 * g + 8 * (i & 1);  // multiple of 8: byte offset of the piece
  intx8 out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 32 * h + 8 * r + (i >> 1);
    const int c = col >> 4;
    const int off = row * (A_LIKE ? ROW_A : ROW_B) + 16 * (c ^ (A_LIKE ? swz_a(row) : swz_b(row))) + (col & 15);
    const v2i32 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(FORGE_LDS(v2i32, panel + off));
    out[2 * r] = x[0];
    out[2 * r + 1] = x[1];
  }
  return out;
}

__device__ __forceinline__ void mma_stage(floatx16 (&acc)[4][2], const unsigned char* stage, int wm, int wn) {
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + PANEL_A;
  intx8 b[2];
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) b[bj] = frag<false>(pb, wn * 64 + 32 * bj);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const intx8 a = frag<true>(pa, 128 * (bi >> 1) + 64 * wm + 32 * (bi & 1));
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[bj], acc[bi][bj], 0, 0, 0, 127, 0, 127);
  }
}

// acc = sum over all T tokens of dY8[t, n] X8[t, k] (codes, unscaled) for tile (n0, k0).
// Ends with a barrier (LDS free for reuse).
__device__ __forceinline__ void contract(floatx16 (&acc)[4][2], unsigned char* smem, const GemmArgs& g, int n0,
                                         int k0) {
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;
  Feed f;
  make_feed(f, g.dY, g.X, g.T, g.N, g.K, n0, k0);
  const int nsl = (int)((g.T + TK - 1) / TK);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nsl) issue(f, smem + s * STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    const int ahead = min(nsl - 1 - s, STAGES - 2);
    if (ahead >= 1) wait_vm<DMA>();
    else wait_vm<0>();
    barrier();
    if (s + STAGES - 1 < nsl) issue(f, smem + ((s + STAGES - 1) % STAGES) * STAGE, s + STAGES - 1);
    mma_stage(acc, smem + (s % STAGES) * STAGE, wm, wn);
  }
  barrier();
}

// ------------------------------------------------------------------ wide tiles (256 x 256)
// One workgroup of 8 waves contracts a 256 x 256 tile: waves 0-3 the columns k0 .. k0 + 127 and
// waves 4-7 the columns k0 + 128 .. k0 + 255, each with the wave layout above.  Both groups read
// the same dY slab; the X slab is 64 token rows of 256 bytes, laid out and swizzled like dY.  A
// slab moves 32 KiB (one third less than two 256 x 128 tiles) and 4 stages fit in 128 KiB.
// The per-element token order is that of the 256 x 128 path, so the sums are bitwise equal.
constexpr int W_STAGES = 4, W_PANEL = TK * ROW_A, W_STAGE = 2 * W_PANEL, W_SMEM = W_STAGES * W_STAGE;
constexpr int W_DMA = 4;  // per wave per slab: 2 of dY, 2 of X

struct WideFeed {
  u32x4 rA, rB;
  uint32_t offA[2], offB[2];
  uint32_t stepA, stepB;
};

// A 1 KiB DMA covers 4 token rows of 256 bytes; wave w moves rows 8 w .. 8 w + 7 of each panel.
__device__ __forceinline__ void make_wide_feed(WideFeed& f, const GemmArgs& g, int n0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(g.dY, (uint32_t)(g.T * g.N));
  f.rB = make_rsrc(g.X, (uint32_t)(g.T * g.K));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 4 * (2 * wave + j) + (lane >> 4), p = lane & 15;
    f.offA[j] = (uint32_t)(r * g.N + n0 + 16 * (p ^ swz_a(r)));
    f.offB[j] = (uint32_t)(r * g.K + k0 + 16 * (p ^ swz_a(r)));
  }
  f.stepA = (uint32_t)(TK * g.N);
  f.stepB = (uint32_t)(TK * g.K);
}

__device__ __forceinline__ void wide_issue(const WideFeed& f, unsigned char* stage, int slab) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(f.rA, f.offA[j] + sa, stage + (2 * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(f.rB, f.offB[j] + sb, stage + W_PANEL + (2 * wave + j) * 1024);
}

__device__ __forceinline__ void wide_mma_stage(floatx16 (&acc)[4][2], const unsigned char* stage, int wm, int wn,
                                               int kh) {
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + W_PANEL;
  intx8 b[2];
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) b[bj] = frag<false, true>(pb, kh * 128 + wn * 64 + 32 * bj);
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    const intx8 a = frag<true>(pa, 128 * (bi >> 1) + 64 * wm + 32 * (bi & 1));
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
      acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[bj], acc[bi][bj], 0, 0, 0, 127, 0, 127);
  }
}

// acc = this wave's part of the codes' product sum for the 256 x 256 tile at (n0, k0).  Ends
// with a barrier (LDS free for reuse).
__device__ __forceinline__ void contract_wide(floatx16 (&acc)[4][2], unsigned char* smem, const GemmArgs& g, int n0,
                                              int k0) {
  const int wave = threadIdx.x >> 6, kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bj][v] = 0.f;
  WideFeed f;
  make_wide_feed(f, g, n0, k0);
  const int nsl = (int)((g.T + TK - 1) / TK);
#pragma unroll
  for (int s = 0; s < W_STAGES - 1; ++s)
    if (s < nsl) wide_issue(f, smem + s * W_STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    const int ahead = min(nsl - 1 - s, W_STAGES - 2);
    if (ahead >= 2) wait_vm<2 * W_DMA>();
    else if (ahead == 1) wait_vm<W_DMA>();
    else wait_vm<0>();
    barrier();
    if (s + W_STAGES - 1 < nsl) wide_issue(f, smem + ((s + W_STAGES - 1) % W_STAGES) * W_STAGE, s + W_STAGES - 1);
    wide_mma_stage(acc, smem + (s % W_STAGES) * W_STAGE, wm, wn, kh);
  }
  barrier();
}

// Stage rows [half * 128, half * 128 + 128) of the tile's accumulators in LDS as fp32
// [128][EPI_LD], times `scale`.  A wave's 32-row blocks bi are rows 128 (bi / 2) + 64 wm +
// 32 (bi % 2) of the tile (two in each half, so each half frees half of every wave's
// accumulators).  32 x 32 output layout: register v of lane l holds row 8 (v / 4) + 4 (l / 32) +
// v % 4, column l % 32 of its block.
__device__ __forceinline__ void stage_acc_half(float* st, const floatx16 (&acc)[4][2], float scale, int half) {
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const int wm = wave >> 1, wn = wave & 1, c32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (hb != half) continue;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int bj = 0; bj < 2; ++bj)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          st[(64 * wm + 32 * b2 + 8 * (v >> 2) + 4 * h + (v & 3)) * ml2::EPI_LD + wn * 64 + 32 * bj + c32] =
              acc[2 * hb + b2][bj][v] * scale;
  }
}

}  // namespace ml8
}  // namespace forge
