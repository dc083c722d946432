// forge_mainloop.h -- the token contraction of one S x S weight tile on gfx950 (S = 128, or 64
// for fp32 layers with fewer 128 x 128 tiles than CUs).
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism": for one
// tile of W the kernel accumulates the products of the upstream gradient dY and the input
// X over all tokens in fp32 registers.
//
// dW[n, k] = sum_t dY[t, n] X[t, k].  Both operands are stored token-major (row t holds all
// n or all k), while the matrix cores want each lane to hold consecutive tokens for one n
// (A operand) or one k (B operand).  So each slab of TK tokens is read with coalesced 16-byte
// global loads along n / k, transposed in registers (byte permutes), and written to LDS as
// [n][token] / [k][token] rows of 128 bytes (+16 bytes of padding, which makes both the
// transposing writes and the fragment reads free of bank conflicts).  The slab is double
// buffered: the global loads of slab s+1 are in flight while the MFMAs consume slab s.
//
// Any order of the tokens inside a slab is a valid summation order (the explainer's exactness
// argument: only the order of the sum over tokens differs), so the token order inside an LDS
// row need only be the same for the dY and X panels, which it is by construction.
//
// Workgroup: 256 threads = 4 waves of 64; the S x S tile is split 2 x 2 into S/2 x S/2 wave
// tiles of (S/32) x (S/32) MFMA 16x16 blocks (4 x 4 for S = 128, 2 x 2 for S = 64; with
// S = 64 half of the loading threads fetch a slab, and four workgroups share a CU).  Accumulator
// layout (16x16 MFMA output): lane l, register r of block (i, j) holds W row 16 i + 4 (l / 16)
// + r and column 16 j + (l % 16) of the wave tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "forge_device.h"
#include "forge_plan.h"

namespace forge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kLdsRow = 144;      // bytes per LDS panel row: 128 bytes of tokens + 16 pad
constexpr int kEpiLd = 128 + 4;   // fp32 staging row stride (floats) for the epilogue

// Square tiles of side S (128, or 64 for layers too small to fill the chip): four waves, each
// a (S / 2) x (S / 2) quadrant of NB x NB blocks of 16 x 16.
template <int S>
struct SmallTile {
  static_assert(S == 128 || S == 64, "tile side");
  static constexpr int NB = S / 32;
  static constexpr int PANEL = S * kLdsRow;
  static constexpr int STAGE = 2 * PANEL;    // dY panel + X panel
  static constexpr int SMEM = 2 * STAGE;     // double buffered: 73728 bytes for S = 128
  static constexpr int SEGS = S * S / (kThreads * 16);  // 16-element segments per thread
  static constexpr int SEGS_PER_ROW = S / 16;
  static_assert(S * kEpiLd * 4 <= SMEM, "the staging fits the panels' LDS");
};
constexpr int kSmem = SmallTile<128>::SMEM;

// Per input type: element size, tokens per slab (so that a panel row is 128 bytes),
// and the number of 8-row groups a slab holds.
template <int IN>
struct InT;
template <>
struct InT<FORGE_IN_BF16> {
  static constexpr int ESZ = 2, TK = 64, RG = 8;
};
template <>
struct InT<FORGE_IN_F32> {
  static constexpr int ESZ = 4, TK = 32, RG = 4;
};
template <>
struct InT<FORGE_IN_FP8> {
  static constexpr int ESZ = 1, TK = 128, RG = 16;
};

// Workgroup -> tile mapping (XCD-aware; forge_plan.h).
using plan::tile_coords_at;

__device__ __forceinline__ void tile_coords(int nbN, int nbK, int& nb, int& kb) {
  tile_coords_at((int)blockIdx.x, nbN, nbK, nb, kb);
}

// Transpose an 8-row x 16-byte block (rows = tokens) held in registers into per-column token
// vectors and store them into an LDS panel: column j of this thread's 16-byte chunk goes to
// panel row (chunk * 16 / ESZ + j) at byte offset rg * 8 * ESZ.
template <int IN>
__device__ __forceinline__ void store_transposed(unsigned char* panel, const u32x4 (&in)[8], int ch, int rg) {
  constexpr int ESZ = InT<IN>::ESZ;
  if constexpr (IN == FORGE_IN_BF16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(in[2 * p + 1][j >> 1], in[2 * p][j >> 1], sel);
      *reinterpret_cast<u32x4*>(panel + (ch * 8 + j) * kLdsRow + rg * 16) = o;
    }
  } else if constexpr (IN == FORGE_IN_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 o0, o1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        o0[p] = in[p][j];
        o1[p] = in[4 + p][j];
      }
      unsigned char* dst = panel + (ch * 4 + j) * kLdsRow + rg * 32;
      *reinterpret_cast<u32x4*>(dst) = o0;
      *reinterpret_cast<u32x4*>(dst + 16) = o1;
    }
  } else {  // fp8: 4x4 byte transposes
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    uint32_t o[16][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {      // rows 0..3, rows 4..7
#pragma unroll
      for (int d = 0; d < 4; ++d) {    // dword = columns 4d..4d+3
        const uint32_t a0 = in[4 * h][d], a1 = in[4 * h + 1][d], a2 = in[4 * h + 2][d], a3 = in[4 * h + 3][d];
        const uint32_t p01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);
        const uint32_t p01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);
        const uint32_t p23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
        const uint32_t p23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
        o[4 * d + 0][h] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
        o[4 * d + 1][h] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
        o[4 * d + 2][h] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
        o[4 * d + 3][h] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      u32x2 x;
      x[0] = o[j][0];
      x[1] = o[j][1];
      *reinterpret_cast<u32x2*>(panel + (ch * 16 + j) * kLdsRow + rg * 8) = x;
    }
  }
  (void)ESZ;
}

// One slab of MFMAs for a wave tile of NB x NB blocks of 16 x 16.  sA: dY panel rows (n), sB:
// X panel rows (k).
template <int IN, int NB>
__device__ __forceinline__ void mma_slab(floatx4 (&acc)[NB][NB], const unsigned char* sA, const unsigned char* sB,
                                         int lane) {
  const int r16 = lane & 15, q = lane >> 4;
  if constexpr (IN == FORGE_IN_BF16) {
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      bf16x8 a[NB], b[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(sA + (16 * i + r16) * kLdsRow + kq * 64 + q * 16);
        b[i] = *reinterpret_cast<const bf16x8*>(sB + (16 * i + r16) * kLdsRow + kq * 64 + q * 16);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else if constexpr (IN == FORGE_IN_F32) {
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      floatx4 a[NB], b[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        a[i] = *reinterpret_cast<const floatx4*>(sA + (16 * i + r16) * kLdsRow + kq * 64 + q * 16);
        b[i] = *reinterpret_cast<const floatx4*>(sB + (16 * i + r16) * kLdsRow + kq * 64 + q * 16);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
  } else {  // fp8 e4m3 (OCP), 16x16x128; format 0 = e4m3 for both operands, unit (2^0) block scales
    intx8 a[NB], b[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const unsigned char* pa = sA + (16 * i + r16) * kLdsRow + q * 32;
      const unsigned char* pb = sB + (16 * i + r16) * kLdsRow + q * 32;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(pa), a1 = *reinterpret_cast<const u32x4*>(pa + 16);
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(pb), b1 = *reinterpret_cast<const u32x4*>(pb + 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a[i][c] = a0[c];
        a[i][4 + c] = a1[c];
        b[i][c] = b0[c];
        b[i][4 + c] = b1[c];
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 127, 0, 127);
  }
}

// Accumulate the full gradient of the S x S tile (n0, k0) over all T tokens into acc (per
// wave).  Ends with a barrier, so the caller may reuse the LDS.
template <int IN, int S>
__device__ __forceinline__ void contract_tile(floatx4 (&acc)[SmallTile<S>::NB][SmallTile<S>::NB], unsigned char* smem,
                                              const GemmArgs& g, int n0, int k0) {
  constexpr int ESZ = InT<IN>::ESZ, TK = InT<IN>::TK, RG = InT<IN>::RG;
  constexpr int NB = SmallTile<S>::NB, kPanel = SmallTile<S>::PANEL, kStage = SmallTile<S>::STAGE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // loader role: threads 0..127 fetch the dY panel, 128..255 the X panel; a panel is S * ESZ / 16
  // chunks of 16 bytes times RG groups of 8 tokens (all 128 threads for S = 128, half for S = 64)
  const int op = tid >> 7, lt = tid & 127, rg = lt % RG, ch = lt / RG;
  const bool loader = lt < (S * ESZ / 16) * RG;
  const unsigned char* src = op ? static_cast<const unsigned char*>(g.X) + (int64_t)k0 * ESZ
                                : static_cast<const unsigned char*>(g.dY) + (int64_t)n0 * ESZ;
  src += ch * 16;
  const int64_t rstride = (op ? g.K : g.N) * ESZ;
  const int64_t T = g.T;
  const int nsl = (int)((T + TK - 1) / TK);

  // wave tile: rows wm * S / 2.. of the dY panel, rows wn * S / 2.. of the X panel
  const int wm = wave >> 1, wn = wave & 1;

  u32x4 buf[8];
  auto load = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t t = (int64_t)s * TK + rg * 8 + i;
      buf[i] = t < T ? ld16(src + t * rstride) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  if (nsl > 0 && loader) {
    load(0);
    store_transposed<IN>(smem + op * kPanel, buf, ch, rg);
  }
  __syncthreads();
  for (int s = 0; s < nsl; ++s) {
    unsigned char* stage = smem + (s & 1) * kStage;
    const bool more = s + 1 < nsl && loader;
    if (more) load(s + 1);
    mma_slab<IN, NB>(acc, stage + wm * (S / 2) * kLdsRow, stage + kPanel + wn * (S / 2) * kLdsRow, lane);
    if (more) store_transposed<IN>(smem + ((s + 1) & 1) * kStage + op * kPanel, buf, ch, rg);
    __syncthreads();
  }
}

// Stage the accumulators of the S x S tile in LDS as fp32 [S][kEpiLd], multiplied by `scale`,
// so that each thread can then read 16 consecutive columns of one row.
template <int S>
__device__ __forceinline__ void stage_acc(float* st, const floatx4 (&acc)[SmallTile<S>::NB][SmallTile<S>::NB],
                                          float scale) {
  constexpr int NB = SmallTile<S>::NB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, r16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st[(wm * (S / 2) + 16 * i + 4 * q + r) * kEpiLd + wn * (S / 2) + 16 * j + r16] = acc[i][j][r] * scale;
}

// Row and first column (within the tile) of this thread's segment s of 16 elements.
template <int S>
__device__ __forceinline__ void small_seg(int s, int& row, int& col) {
  const int seg = (int)threadIdx.x + kThreads * s;
  row = seg / SmallTile<S>::SEGS_PER_ROW;
  col = (seg % SmallTile<S>::SEGS_PER_ROW) * 16;
}

__device__ __forceinline__ void read_seg16(float (&g)[16], const float* st, int row, int col) {
  const float* p = st + row * kEpiLd + col;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(p + 4 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) g[4 * q + c] = x[c];
  }
}

}  // namespace forge
