// forge_mainloop2.h -- token contraction of a 256 x 128 weight tile (two 128 x 128 tiles of
// the method) for bf16 inputs, fed by direct global->LDS DMA and LDS transpose reads.
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": the tile's
// gradient dW[n, k] = sum_t dY[t, n] X[t, k] is accumulated over all tokens in fp32
// registers.  Any order of the tokens is a valid summation order (section 2 "Precision and
// Fidelity"), so the token <-> MFMA k-slot assignment only has to be the same for dY and X.
//
// Data path (gfx950):
//  * A slab of TK = 32 tokens of dY[:, n0:n0+256] (16 KiB) and X[:, k0:k0+128] (8 KiB) is
//    copied to LDS by buffer_load_dwordx4 ... lds: every lane moves 16 bytes and the wave's
//    64 lanes fill 1 KiB of LDS in lane order.  Rows stay token-major, exactly as in HBM.
//    Tokens past T read as zero (buffer range check), so a ragged last slab needs no code.
//  * STAGES slabs live in LDS (3 x 24 KiB for full tiles); the copy of slab s + STAGES - 1 is
//    issued while slab s is multiplied.
//  * The MFMA operands need 8 tokens of one n (or k) per lane.  ds_read_b64_tr_b16 gives
//    exactly that from token-major rows: within each group of 16 lanes, lane j receives
//    element (j % 4) of the 8-byte piece addressed by lane 4 f + j / 4, for f = 0..3.  Lane
//    i of a group therefore points at token row (base + i / 4), columns (c0 + 4 (i % 4)) ..
//    +3, and lane j gets tokens base..base+3 of column c0 + j.
//  * 16-byte chunks of a token row are XOR-swizzled with 2 * (t mod 8), chosen through the
//    global address each DMA lane fetches; the transpose reads of 8 consecutive token rows
//    then hit 8 disjoint bank groups.
//
// Workgroup: 256 threads = 4 waves as 2 (n) x 2 (k).  Full tiles are 256 x 128: a wave holds
// 8 x 4 MFMA 16x16x32 blocks (128 accumulator registers per lane) of 64 columns and 128 rows,
// rows 64 wm .. 64 wm + 63 of each 128-row half of the tile (a_row), so that each half of the
// epilogue frees half of every wave's accumulators.  Half tiles are 128 x 128 (wave tile
// 64 x 64) and balance the last round of a launch (see the launcher).  Two workgroups per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "forge_device.h"

namespace forge {
namespace ml2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define FORGE_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int BM = 256, BN = 128, THREADS = 256;   // full tile
constexpr int BM_HALF = 128;                        // half tile
constexpr int ROW_B = BN * 2;          // bytes per X token row (256)
constexpr int EPI_LD = BN + 4;         // fp32 staging row stride (floats)
constexpr int EPI_ROWS = 128;          // the epilogue stages 128 rows of a tile at a time
constexpr int EPI_BYTES = EPI_ROWS * EPI_LD * 4;

// Pipeline shape: TK tokens per slab, STAGES slabs in LDS, MB 16-row MFMA blocks per wave
// (tile height 32 MB: 8 -> 256 rows, 4 -> 128 rows).
template <int TK_, int STAGES_, int MB_ = 8>
struct Pipe {
  static constexpr int TK = TK_, STAGES = STAGES_, MB = MB_;
  static constexpr int TILE_M = 32 * MB;
  static constexpr int ROW_A = TILE_M * 2;                 // bytes per dY token row in LDS
  static constexpr int PANEL_A = TK * ROW_A, PANEL_B = TK * ROW_B;
  static constexpr int STAGE = PANEL_A + PANEL_B;
  static constexpr int SMEM = STAGES * STAGE;
  static constexpr int DMA_A = PANEL_A / 1024 / 4, DMA_B = PANEL_B / 1024 / 4;  // per wave per slab
  static constexpr int DMA = DMA_A + DMA_B;
  static constexpr int CPR_A = ROW_A / 16, RPD_A = 64 / CPR_A;  // 16-byte chunks per row, rows per 1 KiB
  static_assert(TK % 32 == 0 && DMA < 32 && (STAGES == 3 || STAGES == 4), "pipeline shape");
  static_assert((MB == 8 || MB == 4) && DMA_A >= 1, "tile height");
};

__device__ __forceinline__ int swz(int row) { return 2 * (row & 7); }

// s_waitcnt with only the vector-memory counter limited to n (n < 64); lgkm and exp at max.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier that orders LDS use between the waves without waiting for outstanding DMA.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer resource (gfx9 layout): 48-bit base, stride 0, num_records bytes, default format word.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// One 16-byte-per-lane copy global -> LDS (lane l lands at lds + 16 l).  Issued as inline asm
// so that the compiler does not add a wait for it before every LDS read (it cannot prove the
// copy and the reads touch different stages); completion is awaited explicitly with wait_vm.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, const unsigned char* lds) {
  const uint32_t la =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(la), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <class P>
struct Feed {
  u32x4 rA, rB;                           // dY and X as buffer resources (out-of-range reads give 0)
  uint32_t offA[P::DMA_A], offB[P::DMA_B];  // per-lane byte offsets of this wave's DMA pieces, token 0
  uint32_t stepA, stepB;                  // bytes per slab (TK rows)
};

// Per-lane DMA offsets.  A 1 KiB DMA covers RPD_A dY rows (2 of 512 bytes for full tiles, 4 of
// 256 bytes for half tiles) or 4 X rows; wave w moves dY rows RPD_A d .. (d = DMA_A w + j) and
// X rows 4 x .. 4 x + 3 (x = DMA_B w + j).
template <class P>
__device__ __forceinline__ void make_feed(Feed<P>& f, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                                          int n0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(dY, (uint32_t)(T * N * 2));
  f.rB = make_rsrc(X, (uint32_t)(T * K * 2));
#pragma unroll
  for (int j = 0; j < P::DMA_A; ++j) {
    const int d = P::DMA_A * wave + j, r = P::RPD_A * d + lane / P::CPR_A, p = lane % P::CPR_A;
    const int c = p ^ swz(r);
    f.offA[j] = (uint32_t)(r * N * 2 + n0 * 2 + c * 16);
  }
#pragma unroll
  for (int j = 0; j < P::DMA_B; ++j) {
    const int x = P::DMA_B * wave + j, r = 4 * x + (lane >> 4), p = lane & 15;
    const int c = p ^ swz(r);
    f.offB[j] = (uint32_t)(r * K * 2 + k0 * 2 + c * 16);
  }
  f.stepA = (uint32_t)(P::TK * N * 2);
  f.stepB = (uint32_t)(P::TK * K * 2);
}

template <class P>
__device__ __forceinline__ void issue(const Feed<P>& f, unsigned char* stage, int slab) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < P::DMA_A; ++j) dma16(f.rA, f.offA[j] + sa, stage + (P::DMA_A * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < P::DMA_B; ++j) dma16(f.rB, f.offB[j] + sb, stage + P::PANEL_A + (P::DMA_B * wave + j) * 1024);
}

// Byte offset (within a panel) of this lane's transpose-read piece for 16 columns starting at
// c0, token rows base + (lane % 16) / 4 of a 32-token step.
__device__ __forceinline__ int tr_off(int row_bytes, int row, int c0, int i) {
  const int c = (c0 >> 3) + ((i & 3) >> 1);
  return row * row_bytes + 16 * (c ^ swz(row)) + 8 * (i & 1);
}

__device__ __forceinline__ bf16x8 frag(const unsigned char* panel, int row_bytes, int r0, int r1, int c0, int i) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FORGE_LDS(v4i16, panel + tr_off(row_bytes, r0, c0, i)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FORGE_LDS(v4i16, panel + tr_off(row_bytes, r1, c0, i)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}

// Tile row of a wave's MFMA row block bi.  Full tiles (MB = 8): the wave's 8 blocks are two
// groups of 4, one in each 128-row half of the tile (rows 64 wm .. of each half), so that each
// half of the epilogue stages 4 blocks of every wave and frees their registers.  Half tiles
// (MB = 4): rows 64 wm + 16 bi.
template <int MB>
__device__ __forceinline__ int a_row(int wm, int bi) {
  if constexpr (MB == 8) return 128 * (bi >> 2) + 64 * wm + 16 * (bi & 3);
  return 64 * wm + 16 * bi;
}

template <class P>
__device__ __forceinline__ void mma_stage(floatx4 (&acc)[P::MB][4], const unsigned char* stage, int wm, int wn) {
  const int lane = threadIdx.x & 63, q = lane >> 4, i = lane & 15;
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + P::PANEL_A;
#pragma unroll
  for (int kk = 0; kk < P::TK / 32; ++kk) {
    const int r0 = 32 * kk + 4 * q + (i >> 2), r1 = r0 + 16;
    bf16x8 b[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) b[bj] = frag(pb, ROW_B, r0, r1, wn * 64 + 16 * bj, i);
#pragma unroll
    for (int bi = 0; bi < P::MB; ++bi) {
      const bf16x8 a = frag(pa, P::ROW_A, r0, r1, a_row<P::MB>(wm, bi), i);
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[bj], acc[bi][bj], 0, 0, 0);
    }
  }
}

// acc = dW of tile (n0, k0) over all T tokens.  STAGES - 1 slabs are in flight ahead of the
// one being multiplied.  Ends with a barrier (LDS free for reuse).
template <class P>
__device__ __forceinline__ void contract(floatx4 (&acc)[P::MB][4], unsigned char* smem, const GemmArgs& g, int n0,
                                         int k0) {
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < P::MB; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = floatx4{0.f, 0.f, 0.f, 0.f};
  Feed<P> f;
  make_feed<P>(f, g.dY, g.X, g.T, g.N, g.K, n0, k0);
  const int nsl = (int)((g.T + P::TK - 1) / P::TK);
#pragma unroll
  for (int s = 0; s < P::STAGES - 1; ++s)
    if (s < nsl) issue<P>(f, smem + s * P::STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    // slabs s+1 .. s+STAGES-2 may still be in flight; slab s must have landed
    const int ahead = min(nsl - 1 - s, P::STAGES - 2);
    if constexpr (P::STAGES == 3) {
      if (ahead >= 1) wait_vm<P::DMA>();
      else wait_vm<0>();
    } else {
      if (ahead >= 2) wait_vm<2 * P::DMA>();
      else if (ahead == 1) wait_vm<P::DMA>();
      else wait_vm<0>();
    }
    barrier();
    if (s + P::STAGES - 1 < nsl) issue<P>(f, smem + ((s + P::STAGES - 1) % P::STAGES) * P::STAGE, s + P::STAGES - 1);
    mma_stage<P>(acc, smem + (s % P::STAGES) * P::STAGE, wm, wn);
  }
  barrier();
}

// ------------------------------------------------------------------ wide tiles (256 x 256)
// One workgroup of 8 waves contracts a 256 x 256 tile: waves 0-3 the columns k0 .. k0 + 127
// and waves 4-7 the columns k0 + 128 .. k0 + 255, each group with the wave layout of the
// 256 x 128 tile above.  Both groups read the same dY panel, so a slab moves 16 KiB of dY and
// 16 KiB of X (one third less than two 256 x 128 tiles), and 4 stages fit in 128 KiB.
// Half-wide tiles (128 x 256, MB = 4) have the same layout with the half tile's 64 x 64 wave
// tiles: 8 KiB of dY and 16 KiB of X per slab.  Every element's sum runs over the tokens in
// the same slab and k-slot order as on the 256 x 128 path, so all give bitwise the same
// gradient.
template <int MB_>
struct WidePipeT {
  static constexpr int MB = MB_, TK = 32, STAGES = 4;
  static constexpr int ROW_A = 64 * MB, ROW_B = 512;  // bytes per dY / X token row in LDS
  static constexpr int PANEL_A = TK * ROW_A, PANEL_B = TK * ROW_B;
  static constexpr int STAGE = PANEL_A + PANEL_B, SMEM = STAGES * STAGE;
  static constexpr int DMA_A = PANEL_A / 8192, DMA_B = PANEL_B / 8192;  // 1 KiB copies per wave per slab
  static constexpr int DMA = DMA_A + DMA_B;
  static constexpr int CPR_A = ROW_A / 16, RPD_A = 64 / CPR_A;  // 16-byte chunks per dY row, rows per copy
  static_assert(MB == 8 || MB == 4, "tile height");
};
using WidePipe = WidePipeT<8>;
using WideHalfPipe = WidePipeT<4>;

template <class P>
struct WideFeed {
  u32x4 rA, rB;
  uint32_t offA[P::DMA_A], offB[P::DMA_B];
  uint32_t stepA, stepB;
};

// A 1 KiB copy covers RPD_A dY rows (2 of 512 bytes, or 4 of 256 bytes for half-wide tiles)
// or 2 X rows of 512 bytes; wave w moves dY rows RPD_A d .. (d = DMA_A w + j) and X rows
// 2 x, 2 x + 1 (x = 2 w + j).  Chunks are XOR-swizzled with 2 (t mod 8) as above.
template <class P>
__device__ __forceinline__ void make_wide_feed(WideFeed<P>& f, const GemmArgs& g, int n0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(g.dY, (uint32_t)(g.T * g.N * 2));
  f.rB = make_rsrc(g.X, (uint32_t)(g.T * g.K * 2));
#pragma unroll
  for (int j = 0; j < P::DMA_A; ++j) {
    const int d = P::DMA_A * wave + j, r = P::RPD_A * d + lane / P::CPR_A, c = (lane % P::CPR_A) ^ swz(r);
    f.offA[j] = (uint32_t)(r * g.N * 2 + n0 * 2 + c * 16);
  }
#pragma unroll
  for (int j = 0; j < P::DMA_B; ++j) {
    const int r = 2 * (P::DMA_B * wave + j) + (lane >> 5), c = (lane & 31) ^ swz(r);
    f.offB[j] = (uint32_t)(r * g.K * 2 + k0 * 2 + c * 16);
  }
  f.stepA = (uint32_t)(P::TK * g.N * 2);
  f.stepB = (uint32_t)(P::TK * g.K * 2);
}

template <class P>
__device__ __forceinline__ void wide_issue(const WideFeed<P>& f, unsigned char* stage, int slab) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < P::DMA_A; ++j) dma16(f.rA, f.offA[j] + sa, stage + (P::DMA_A * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < P::DMA_B; ++j) dma16(f.rB, f.offB[j] + sb, stage + P::PANEL_A + (P::DMA_B * wave + j) * 1024);
}

// The 256 x 128 (or 128 x 128) tile's slab step on 512-byte X rows; kh selects the 128-column
// half of X.
template <class P>
__device__ __forceinline__ void wide_mma_stage(floatx4 (&acc)[P::MB][4], const unsigned char* stage, int wm, int wn,
                                               int kh) {
  const int lane = threadIdx.x & 63, q = lane >> 4, i = lane & 15;
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + P::PANEL_A;
  const int r0 = 4 * q + (i >> 2), r1 = r0 + 16;
  bf16x8 b[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) b[bj] = frag(pb, P::ROW_B, r0, r1, kh * 128 + wn * 64 + 16 * bj, i);
#pragma unroll
  for (int bi = 0; bi < P::MB; ++bi) {
    const bf16x8 a = frag(pa, P::ROW_A, r0, r1, a_row<P::MB>(wm, bi), i);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[bj], acc[bi][bj], 0, 0, 0);
  }
}

// acc = this wave's part of dW for the 256 x 256 (or 128 x 256) tile at (n0, k0).  Ends with
// a barrier.
template <class P>
__device__ __forceinline__ void contract_wide(floatx4 (&acc)[P::MB][4], unsigned char* smem, const GemmArgs& g, int n0,
                                              int k0) {
  const int wave = threadIdx.x >> 6, kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < P::MB; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = floatx4{0.f, 0.f, 0.f, 0.f};
  WideFeed<P> f;
  make_wide_feed<P>(f, g, n0, k0);
  const int nsl = (int)((g.T + P::TK - 1) / P::TK);
#pragma unroll
  for (int s = 0; s < P::STAGES - 1; ++s)
    if (s < nsl) wide_issue<P>(f, smem + s * P::STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    const int ahead = min(nsl - 1 - s, P::STAGES - 2);
    if (ahead >= 2) wait_vm<2 * P::DMA>();
    else if (ahead == 1) wait_vm<P::DMA>();
    else wait_vm<0>();
    barrier();
    if (s + P::STAGES - 1 < nsl) wide_issue<P>(f, smem + ((s + P::STAGES - 1) % P::STAGES) * P::STAGE, s + P::STAGES - 1);
    wide_mma_stage<P>(acc, smem + (s % P::STAGES) * P::STAGE, wm, wn, kh);
  }
  barrier();
}

// Stage rows [half * 128, half * 128 + 128) of the tile's accumulators in LDS as fp32
// [128][EPI_LD], multiplied by `scale`: every wave writes its blocks 4 half .. 4 half + 3.  In
// an 8-wave workgroup each group of 4 waves stages its 128 columns into its own buffer.
__device__ __forceinline__ void stage_acc_half(float* st, const floatx4 (&acc)[8][4], float scale, int half) {
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const int wm = wave >> 1, wn = wave & 1, r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    if (hb != half) continue;
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[(64 * wm + 16 * b4 + 4 * q + r) * EPI_LD + wn * 64 + 16 * bj + r16] = acc[4 * hb + b4][bj][r] * scale;
  }
}

// Stage all 128 rows of a half tile's accumulators in LDS as fp32 [128][EPI_LD], times `scale`
// (in an 8-wave workgroup, each group of 4 waves into its own buffer).
__device__ __forceinline__ void stage_acc_all(float* st, const floatx4 (&acc)[4][4], float scale) {
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const int wm = wave >> 1, wn = wave & 1, r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st[(wm * 64 + 16 * bi + 4 * q + r) * EPI_LD + wn * 64 + 16 * bj + r16] = acc[bi][bj][r] * scale;
}


// ------------------------------------------------------------------ input gradient (dgrad)
// dX[t, k] = sum_n dY[t, n] W[n, k] for a 256-token x 128-column tile, reduced over n in
// slabs of TK = 32.  Same data path as the weight gradient with the roles moved:
//  * the W slab (32 rows of n, 256 bytes each) is the transposed operand, read exactly like
//    the X panel above (lane (q, j) of an MFMA fragment holds n = 4q..4q+3 and 16+4q..+3 of
//    column j);
//  * the dY slab is already reduction-contiguous: 256 token rows of 64 bytes.  A fragment
//    needs, per token, the same n order, i.e. two 8-byte pieces at bytes 8q and 32 + 8q of
//    the row, read with ds_read_b64.  The 16-byte chunks of a row are XOR-swizzled with
//    (row / 4) mod 4, so the 16 rows read by a lane group fall in 16 distinct bank windows.
struct DgradPipe {
  static constexpr int TK = 32, STAGES = 3;
  static constexpr int ROW_D = TK * 2;                   // dY bytes per token row in LDS (64)
  static constexpr int PANEL_A = 256 * ROW_D;            // 16 KiB
  static constexpr int PANEL_B = TK * ROW_B;             // 8 KiB
  static constexpr int STAGE = PANEL_A + PANEL_B, SMEM = STAGES * STAGE;
  static constexpr int DMA_A = PANEL_A / 1024 / 4, DMA_B = PANEL_B / 1024 / 4, DMA = DMA_A + DMA_B;
};

__device__ __forceinline__ int swz_d(int row) { return (row >> 2) & 3; }

struct DgradFeed {
  u32x4 rA, rB;
  uint32_t offA[DgradPipe::DMA_A], offB[DgradPipe::DMA_B];
  uint32_t stepA, stepB;
};

// A 1 KiB DMA covers 16 dY token rows (4 chunks each) or 4 W rows (16 chunks each).
__device__ __forceinline__ void make_dgrad_feed(DgradFeed& f, const void* dY, const void* W, int64_t T, int64_t N,
                                                int64_t K, int64_t t0, int k0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(dY, (uint32_t)(T * N * 2));
  f.rB = make_rsrc(W, (uint32_t)(N * K * 2));
#pragma unroll
  for (int j = 0; j < DgradPipe::DMA_A; ++j) {
    const int d = DgradPipe::DMA_A * wave + j, r = 16 * d + (lane >> 2), p = lane & 3;
    f.offA[j] = (uint32_t)((t0 + r) * N * 2 + 16 * (p ^ swz_d(r)));
  }
#pragma unroll
  for (int j = 0; j < DgradPipe::DMA_B; ++j) {
    const int x = DgradPipe::DMA_B * wave + j, r = 4 * x + (lane >> 4), p = lane & 15;
    f.offB[j] = (uint32_t)(r * K * 2 + k0 * 2 + 16 * (p ^ swz(r)));
  }
  f.stepA = (uint32_t)(DgradPipe::TK * 2);
  f.stepB = (uint32_t)(DgradPipe::TK * K * 2);
}

__device__ __forceinline__ void dgrad_issue(const DgradFeed& f, unsigned char* stage, int slab) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < DgradPipe::DMA_A; ++j)
    dma16(f.rA, f.offA[j] + sa, stage + (DgradPipe::DMA_A * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < DgradPipe::DMA_B; ++j)
    dma16(f.rB, f.offB[j] + sb, stage + DgradPipe::PANEL_A + (DgradPipe::DMA_B * wave + j) * 1024);
}

// dY fragment of token rows row0 .. row0 + 15 for lane group q: n = 4q..4q+3, 16+4q..+3.
__device__ __forceinline__ bf16x8 dy_frag(const unsigned char* panel, int row, int q) {
  auto piece = [&](int byte) {
    const int c = byte >> 4;
    return *reinterpret_cast<const v4i16*>(panel + row * DgradPipe::ROW_D + 16 * (c ^ swz_d(row)) + (byte & 15));
  };
  const v4i16 lo = piece(8 * q), hi = piece(32 + 8 * q);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ void dgrad_mma_stage(floatx4 (&acc)[8][4], const unsigned char* stage, int wm, int wn) {
  const int lane = threadIdx.x & 63, q = lane >> 4, i = lane & 15;
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + DgradPipe::PANEL_A;
  const int r0 = 4 * q + (i >> 2), r1 = r0 + 16;
  bf16x8 b[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) b[bj] = frag(pb, ROW_B, r0, r1, wn * 64 + 16 * bj, i);
#pragma unroll
  for (int bi = 0; bi < 8; ++bi) {
    const bf16x8 a = dy_frag(pa, a_row<8>(wm, bi) + i, q);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[bj], acc[bi][bj], 0, 0, 0);
  }
}

// acc = dX of tile (t0, k0) over all n.  Same pipelining as contract().
__device__ __forceinline__ void dgrad_contract(floatx4 (&acc)[8][4], unsigned char* smem, const void* dY, const void* W,
                                               int64_t T, int64_t N, int64_t K, int64_t t0, int k0) {
  using P = DgradPipe;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < 8; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = floatx4{0.f, 0.f, 0.f, 0.f};
  DgradFeed f;
  make_dgrad_feed(f, dY, W, T, N, K, t0, k0);
  const int nsl = (int)(N / P::TK);
#pragma unroll
  for (int s = 0; s < P::STAGES - 1; ++s)
    if (s < nsl) dgrad_issue(f, smem + s * P::STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    const int ahead = min(nsl - 1 - s, P::STAGES - 2);
    if (ahead >= 1) wait_vm<P::DMA>();
    else wait_vm<0>();
    barrier();
    if (s + P::STAGES - 1 < nsl) dgrad_issue(f, smem + ((s + P::STAGES - 1) % P::STAGES) * P::STAGE, s + P::STAGES - 1);
    dgrad_mma_stage(acc, smem + (s % P::STAGES) * P::STAGE, wm, wn);
  }
  barrier();
}

// ------------------------------------------------------------------ wide dgrad tiles
// dX tiles of 256 tokens x 256 columns in one workgroup of 8 waves: waves 0-3 compute columns
// k0 .. k0 + 127 and waves 4-7 columns k0 + 128 .. k0 + 255, each with the wave layout above.
// Both halves read the same dY slab (256 token rows of 32 n), so a slab moves 16 KiB of dY and
// 16 KiB of W (32 rows of 256 columns) and 4 stages fit in 128 KiB.  Every element's sum runs
// over n in the same order as on the 256 x 128 path, so both give bitwise the same dX.
struct DgradWidePipe {
  static constexpr int TK = 32, STAGES = 4;
  static constexpr int ROW_D = TK * 2;                   // dY bytes per token row (64)
  static constexpr int ROW_W = 512;                      // W bytes per row of n (256 columns)
  static constexpr int PANEL_A = 256 * ROW_D, PANEL_B = TK * ROW_W;   // 16 KiB each
  static constexpr int STAGE = PANEL_A + PANEL_B, SMEM = STAGES * STAGE;
  static constexpr int DMA = 4;                          // per wave per slab: 2 of dY, 2 of W
};

struct DgradWideFeed {
  u32x4 rA, rB;
  uint32_t offA[2], offB[2];
  uint32_t stepA, stepB;
};

// Wave w (0..7) moves dY token rows 32 w .. 32 w + 31 (a 1 KiB DMA is 16 rows of 4 chunks) and
// W rows 4 w .. 4 w + 3 (a 1 KiB DMA is 2 rows of 32 chunks).
__device__ __forceinline__ void make_dgrad_wide_feed(DgradWideFeed& f, const void* dY, const void* W, int64_t T,
                                                     int64_t N, int64_t K, int64_t t0, int k0) {
  using P = DgradWidePipe;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f.rA = make_rsrc(dY, (uint32_t)(T * N * 2));
  f.rB = make_rsrc(W, (uint32_t)(N * K * 2));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ra = 16 * (2 * wave + j) + (lane >> 2), pa = lane & 3;
    f.offA[j] = (uint32_t)((t0 + ra) * N * 2 + 16 * (pa ^ swz_d(ra)));
    const int rb = 2 * (2 * wave + j) + (lane >> 5), pb = lane & 31;
    f.offB[j] = (uint32_t)(rb * K * 2 + k0 * 2 + 16 * (pb ^ swz(rb)));
  }
  f.stepA = (uint32_t)(P::TK * 2);
  f.stepB = (uint32_t)(P::TK * K * 2);
}

__device__ __forceinline__ void dgrad_wide_issue(const DgradWideFeed& f, unsigned char* stage, int slab) {
  using P = DgradWidePipe;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t sa = (uint32_t)slab * f.stepA, sb = (uint32_t)slab * f.stepB;
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(f.rA, f.offA[j] + sa, stage + (2 * wave + j) * 1024);
#pragma unroll
  for (int j = 0; j < 2; ++j) dma16(f.rB, f.offB[j] + sb, stage + P::PANEL_A + (2 * wave + j) * 1024);
}

__device__ __forceinline__ void dgrad_wide_mma_stage(floatx4 (&acc)[8][4], const unsigned char* stage, int wm,
                                                     int wn, int kh) {
  using P = DgradWidePipe;
  const int lane = threadIdx.x & 63, q = lane >> 4, i = lane & 15;
  const unsigned char* pa = stage;
  const unsigned char* pb = stage + P::PANEL_A;
  const int r0 = 4 * q + (i >> 2), r1 = r0 + 16;
  bf16x8 b[4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj) b[bj] = frag(pb, P::ROW_W, r0, r1, kh * 128 + wn * 64 + 16 * bj, i);
#pragma unroll
  for (int bi = 0; bi < 8; ++bi) {
    const bf16x8 a = dy_frag(pa, a_row<8>(wm, bi) + i, q);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[bj], acc[bi][bj], 0, 0, 0);
  }
}

// acc = this wave's part of dX for the 256-token x 256-column tile at (t0, k0).  Ends with a
// barrier (LDS free for reuse).
__device__ __forceinline__ void dgrad_wide_contract(floatx4 (&acc)[8][4], unsigned char* smem, const void* dY,
                                                    const void* W, int64_t T, int64_t N, int64_t K, int64_t t0,
                                                    int k0) {
  using P = DgradWidePipe;
  const int wave = threadIdx.x >> 6, kh = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
#pragma unroll
  for (int bi = 0; bi < 8; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = floatx4{0.f, 0.f, 0.f, 0.f};
  DgradWideFeed f;
  make_dgrad_wide_feed(f, dY, W, T, N, K, t0, k0);
  const int nsl = (int)(N / P::TK);
#pragma unroll
  for (int s = 0; s < P::STAGES - 1; ++s)
    if (s < nsl) dgrad_wide_issue(f, smem + s * P::STAGE, s);
  for (int s = 0; s < nsl; ++s) {
    const int ahead = min(nsl - 1 - s, P::STAGES - 2);
    if (ahead >= 2) wait_vm<2 * P::DMA>();
    else if (ahead == 1) wait_vm<P::DMA>();
    else wait_vm<0>();
    barrier();
    if (s + P::STAGES - 1 < nsl) dgrad_wide_issue(f, smem + ((s + P::STAGES - 1) % P::STAGES) * P::STAGE, s + P::STAGES - 1);
    dgrad_wide_mma_stage(acc, smem + (s % P::STAGES) * P::STAGE, wm, wn, kh);
  }
  barrier();
}

}  // namespace ml2
}  // namespace forge
