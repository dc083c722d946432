// forge_kernels.hip -- kernels and launchers of the fused and the unfused paths.
//
// Fused (FORGE explainer, gist.science, Technical Summary section 2 "Core Mechanism"): one
// workgroup per tile of W contracts dY and X over all tokens into fp32 accumulators, then
// applies the optimizer to the tile and writes back only W and its moments.  The gradient
// tile lives in registers and, for the re-layout to 16 consecutive columns per thread, in the
// workgroup's LDS; it never reaches HBM.  Three contraction paths, chosen per call:
//   * bf16 inputs: 256 x 128 tiles (two of the method's 128 x 128 tiles) fed by LDS DMA,
//     two workgroups per CU, with 128 x 128 half tiles balancing the last round of the launch
//     (forge_mainloop2.h); for T >= 8192, 256 x 256 tiles in one 8-wave workgroup per CU
//     where they fill whole rounds, the remaining columns in a second 256 x 128 launch;
//   * fp8 e4m3 inputs: the same tiles with 8-bit transpose reads (forge_mainloop8.h);
//   * fp32 inputs and layers with too few tiles: 128 x 128 tiles staged through registers
//     (forge_mainloop.h).
// The element-wise update of a 16-element segment (forge_device.h) is shared by all of them.
//
// Unfused baseline (Technical Summary section 1 "The Problem"): the same contraction writes
// the fp32 gradient to HBM, and a separate element-wise kernel reads it back and applies the
// same update code.
//
// dgrad: dX = dY W on the LDS-DMA path (256-token x 256-column tiles in one 8-wave workgroup
// per CU where K % 256 == 0 and they fill the CUs, else 256 x 128), run before the step so
// that it sees the old weight (Technical Summary section 5, limitations).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "forge_mainloop.h"
#include "forge_mainloop2.h"
#include "forge_mainloop8.h"

namespace forge {

template <int IN>
__device__ __forceinline__ float input_scale(const GemmArgs& g) {
  if constexpr (IN == FORGE_IN_FP8) return g.dy_scale[0] * g.x_scale[0];
  return 1.0f;
}

template <int IN, int WT, int ST, int OPT>
__global__ __launch_bounds__(kThreads, 2) void fused_step_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  const int nbN = (int)(g.N / kBM), nbK = (int)(g.K / kBN);
  int nb, kb;
  tile_coords(nbN, nbK, nb, kb);
  const int n0 = nb * kBM, k0 = kb * kBN;

  floatx4 acc[4][4];
  contract_tile<IN>(acc, smem, g, n0, k0);

  float* st = reinterpret_cast<float*>(smem);
  stage_acc(st, acc, input_scale<IN>(g));
  __syncthreads();
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int s = 0; s < 4; ++s) {
    const int seg = tid + kThreads * s, row = seg >> 3, kseg = seg & 7;
    float gr[16];
    read_seg16(gr, st, row, kseg);
    const uint32_t i0 = (uint32_t)(n0 + row) * (uint32_t)g.K + (uint32_t)(k0 + kseg * 16);
    step_segment16<OPT, WT, ST>(gr, i0, e);
  }
}

template <int IN>
__global__ __launch_bounds__(kThreads, 2) void wgrad_gemm_kernel(GemmArgs g, float* dW) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  const int nbN = (int)(g.N / kBM), nbK = (int)(g.K / kBN);
  int nb, kb;
  tile_coords(nbN, nbK, nb, kb);
  const int n0 = nb * kBM, k0 = kb * kBN;

  floatx4 acc[4][4];
  contract_tile<IN>(acc, smem, g, n0, k0);

  float* st = reinterpret_cast<float*>(smem);
  stage_acc(st, acc, input_scale<IN>(g));
  __syncthreads();
  const int tid = threadIdx.x;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int seg = tid + kThreads * s, row = seg >> 3, kseg = seg & 7;
    const float* p = st + row * kEpiLd + kseg * 16;
    float* d = dW + (int64_t)(n0 + row) * g.K + k0 + kseg * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(d + 4 * q, *reinterpret_cast<const u32x4*>(p + 4 * q));
  }
}

// bf16 inputs, 256 x 128 workgroup tiles fed by LDS DMA (forge_mainloop2.h): 32-token slabs,
// three in LDS (72 KiB), so two workgroups share a CU and each SIMD runs two waves.  The
// launcher may turn the last k-block columns into 128 x 128 half tiles (four 32-token slabs in
// LDS) so that the last round of workgroups fills the chip (see plan_split).
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

// Full 256 x 128 tile.  Epilogue: the gradient goes through LDS in two 128-row halves; each
// thread owns 4 segments of 16 elements per half.  The stored state of the next two segments
// is in flight while the current one is updated (the first loads leave before the staging);
// in the first half the other half's accumulators are still live, so unless DEEP0 only one
// segment is in flight there (bf16 weights with fp32 moments on the bf16 path use two).
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
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    stage(h);
    __syncthreads();
    batch(xa, xb, h, 0);
    batch(xb, xa, h, 1);
    batch(xa, xb, h, 2);
    batch(xb, xa, h, 3);
    __syncthreads();
  }
}

// Segment epilogue: 16 consecutive elements of a row per thread (4 per 128-row half), the
// stored state of the next two segments in flight while one is updated.  Used for int8
// moments: with 1-byte codes and per-block scales the 4-element units take about 3x more
// small memory instructions per element than 16-element segments, and the contiguous-lane
// layout gains little on such narrow data.
template <int OPT, int WT, int ST, int HALVES, class Stage>
__device__ __forceinline__ void seg_epilogue(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                             int k0, Stage&& stage) {
  float* st = reinterpret_cast<float*>(smem);
  auto index_of = [&](int j) {  // the thread's j-th segment (j = 4 half + s)
    int row, kseg;
    seg_pos(j & 3, row, kseg);
    return (uint32_t)(n0 + (j >> 2) * ml2::EPI_ROWS + row) * (uint32_t)g.K + (uint32_t)(k0 + kseg * 16);
  };
  // one segment in flight: the int8 update needs more registers than the fp32 one, and the
  // accumulators of the second half are still live during the first
  SegIn x0;
  seg_load<OPT, WT, ST>(x0, index_of(0), e);
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    stage(h);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int j = 4 * h + s;
      float gr[16];
      staged_grad(st, s, gr);
      seg_apply<OPT, WT, ST>(gr, index_of(j), x0, e);
      if (j + 1 < 4 * HALVES) seg_load<OPT, WT, ST>(x0, index_of(j + 1), e);
    }
    __syncthreads();
  }
}

// The epilogue for the state format: 4-element units for fp32 moments, segments for int8
// (SEG_INT8; the fp8 kernel keeps units for int8, where the segment form does not fit its
// registers).
template <int OPT, int WT, int ST, int HALVES, bool SEG_INT8, class Stage>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int n0,
                                              int k0, Stage&& stage) {
  if constexpr (ST == FORGE_S_Q8 && SEG_INT8) seg_epilogue<OPT, WT, ST, HALVES>(g, e, smem, n0, k0, stage);
  else unit_epilogue<OPT, WT, ST, HALVES>(g, e, smem, n0, k0, stage);
}

// Full 256 x 128 tile: contraction, then the epilogue over its two 128-row halves.
template <int WT, int ST, int OPT>
__device__ __forceinline__ void fused_full_tile(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int b) {
  int nb, kb;
  tile_coords_at(b, (int)(g.N / ml2::BM), g.kb_split, nb, kb);
  const int n0 = nb * ml2::BM, k0 = (g.kb_base + kb) * ml2::BN;
  ml2::floatx4 acc[8][4];
  ml2::contract<Pipe2>(acc, smem, g, n0, k0);
  float* st = reinterpret_cast<float*>(smem);
  tile_epilogue<OPT, WT, ST, 2, true>(g, e, smem, n0, k0, [&](int h) { ml2::stage_acc_half(st, acc, 1.0f, h); });
}

// Half 128 x 128 tile hb of the blocks [kb_split, nbk): all 128 rows staged at once.
template <int WT, int ST, int OPT>
__device__ __forceinline__ void fused_half_tile(const GemmArgs& g, const EpiArgs& e, unsigned char* smem, int hb) {
  int nb, kb;
  tile_coords_at(hb, (int)(g.N / ml2::BM_HALF), g.nbk - g.kb_split, nb, kb);
  const int n0 = nb * ml2::BM_HALF, k0 = (g.kb_base + g.kb_split + kb) * ml2::BN;
  ml2::floatx4 acc[4][4];
  ml2::contract<Pipe2H>(acc, smem, g, n0, k0);
  float* st = reinterpret_cast<float*>(smem);
  tile_epilogue<OPT, WT, ST, 1, true>(g, e, smem, n0, k0, [&](int) { ml2::stage_acc_all(st, acc, 1.0f); });
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
// threads 256-511 columns k0 + 128 .. k0 + 255, each staging through its own LDS buffer.  The
// launch covers the nbk / 2 wide column blocks from kb_base / 2 on.
constexpr int kSmemW = ml2::WidePipe::SMEM > 2 * ml2::EPI_BYTES ? ml2::WidePipe::SMEM : 2 * ml2::EPI_BYTES;
static_assert(kSmemW <= 160 * 1024, "wide tiles fit the CU's LDS");

template <int WT, int ST, int OPT>
__global__ __launch_bounds__(2 * ml2::THREADS, 1) void fused_step_kernel2w(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemW];
  int nb, kb;
  tile_coords_at((int)blockIdx.x, (int)(g.N / ml2::BM), g.nbk / 2, nb, kb);
  const int kh = (int)(threadIdx.x >> 8);
  const int n0 = nb * ml2::BM, kw0 = (g.kb_base + 2 * kb) * ml2::BN;
  ml2::floatx4 acc[8][4];
  ml2::contract_wide(acc, smem, g, n0, kw0);
  unsigned char* mine = smem + kh * ml2::EPI_BYTES;
  float* st = reinterpret_cast<float*>(mine);
  tile_epilogue<OPT, WT, ST, 2, true>(g, e, mine, n0, kw0 + kh * ml2::BN,
                                      [&](int h) { ml2::stage_acc_half(st, acc, 1.0f, h); });
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

__global__ __launch_bounds__(ml2::THREADS, kOcc2) void wgrad_gemm_kernel2(GemmArgs g, float* dW) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  float* st = reinterpret_cast<float*>(smem);
  const int b = (int)blockIdx.x;
  int nb, kb;
  if (b < g.nfull) {
    tile_coords_at(b, (int)(g.N / ml2::BM), g.kb_split, nb, kb);
    const int n0 = nb * ml2::BM, k0 = (g.kb_base + kb) * ml2::BN;
    ml2::floatx4 acc[8][4];
    ml2::contract<Pipe2>(acc, smem, g, n0, k0);
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      ml2::stage_acc_half(st, acc, 1.0f, half);
      __syncthreads();
      store_staged(st, dW, g.K, n0 + half * ml2::EPI_ROWS, k0);
      __syncthreads();
    }
  } else {
    tile_coords_at(b - g.nfull, (int)(g.N / ml2::BM_HALF), g.nbk - g.kb_split, nb, kb);
    const int n0 = nb * ml2::BM_HALF, k0 = (g.kb_base + g.kb_split + kb) * ml2::BN;
    ml2::floatx4 acc[4][4];
    ml2::contract<Pipe2H>(acc, smem, g, n0, k0);
    ml2::stage_acc_all(st, acc, 1.0f);
    __syncthreads();
    store_staged(st, dW, g.K, n0, k0);
  }
}

// fp8 e4m3 inputs, 256 x 128 tiles fed by LDS DMA with 8-bit transpose reads
// (forge_mainloop8.h); the tensors' scale product multiplies the finished sums at staging.
static_assert(ml8::SMEM <= kSmem2, "fp8 stages fit the shared buffer size");

// The launch covers the nbk 128-column blocks from kb_base on.
template <int WT, int ST, int OPT>
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void fused_step_kernel8(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  int nb, kb;
  tile_coords((int)(g.N / ml2::BM), g.nbk, nb, kb);
  const int n0 = nb * ml2::BM, k0 = (g.kb_base + kb) * ml2::BN;
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
  int nb, kb;
  tile_coords_at((int)blockIdx.x, (int)(g.N / ml2::BM), g.nbk / 2, nb, kb);
  const int kh = (int)(threadIdx.x >> 8);
  const int n0 = nb * ml2::BM, kw0 = (g.kb_base + 2 * kb) * ml2::BN;
  ml8::floatx16 acc[4][2];
  ml8::contract_wide(acc, smem, g, n0, kw0);
  const float scale = g.dy_scale[0] * g.x_scale[0];
  unsigned char* mine = smem + kh * ml2::EPI_BYTES;
  float* st = reinterpret_cast<float*>(mine);
  tile_epilogue<OPT, WT, ST, 2, false>(g, e, mine, n0, kw0 + kh * ml2::BN,
                                       [&](int h) { ml8::stage_acc_half(st, acc, scale, h); });
}

__global__ __launch_bounds__(ml2::THREADS, kOcc2) void wgrad_gemm_kernel8(GemmArgs g, float* dW) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  int nb, kb;
  tile_coords((int)(g.N / ml2::BM), (int)(g.K / ml2::BN), nb, kb);
  const int n0 = nb * ml2::BM, k0 = kb * ml2::BN;
  ml8::floatx16 acc[4][2];
  ml8::contract(acc, smem, g, n0, k0);
  const float scale = g.dy_scale[0] * g.x_scale[0];
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    ml8::stage_acc_half(st, acc, scale, half);
    __syncthreads();
    store_staged(st, dW, g.K, n0 + half * ml2::EPI_ROWS, k0);
    __syncthreads();
  }
}

// Workgroup slots on the current device: two 256 x 128 workgroups per CU.
static int slots_on_current_device() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    cached[dev] = 2 * cu;
  }
  return cached[dev];
}

// Tile plan of the 256 x 128 path.  With F full tiles and S workgroup slots, the last round
// holds F mod S tiles and leaves CUs with one workgroup; turning the last c k-block columns
// into 128 x 128 half tiles (c = the fewest columns that hold that remainder) ends the launch
// with a round of half tiles instead.  Returns the grid size.
static unsigned plan_split(GemmArgs& g) {
  const int nbN = (int)(g.N / ml2::BM), nbK = g.nbk;
  const int full = nbN * nbK, slots = slots_on_current_device();
  const int rem = full % slots;
  const int c = rem == 0 ? 0 : std::min(nbK, (rem + nbN - 1) / nbN);
  g.kb_split = nbK - c;
  g.nfull = nbN * g.kb_split;
  return (unsigned)(g.nfull + 2 * nbN * c);
}

// Wide 256 x 256 tiles for long token counts (T >= 8192, where the faster contraction outweighs
// the epilogue that no other workgroup on the CU overlaps; at T = 4096 both layouts take the same
// time): the first kw 256-column blocks of every 256-row block, kw the largest count for which
// N / 256 * kw is a positive multiple of the CU count; 0 otherwise.  The remaining columns run on
// the 256 x 128 path.
static int plan_wide(const GemmArgs& g) {
  if (g.T < 8192) return 0;
  const int nbN = (int)(g.N / ml2::BM), nbK2 = (int)(g.K / (2 * ml2::BN)), cus = slots_on_current_device() / 2;
  for (int kw = nbK2; kw > 0; --kw)
    if ((nbN * kw) % cus == 0) return kw;
  return 0;
}

// The 256 x 128 path needs N % 256 == 0 and at least 128 of its tiles (256 workgroups once the
// plan turns them into half tiles).
static bool use_v2(int in_type, const GemmArgs& g) {
  return in_type == FORGE_IN_BF16 && g.N % ml2::BM == 0 && (g.N / ml2::BM) * (g.K / ml2::BN) >= 128;
}

// fp8 inputs: the DMA path needs N % 256 == 0 and at least 256 of its tiles.
static bool use_v8(int in_type, const GemmArgs& g) {
  return in_type == FORGE_IN_FP8 && g.N % ml2::BM == 0 && (g.N / ml2::BM) * (g.K / ml2::BN) >= 256;
}

// Element-wise rule over a materialised gradient, in the layout of the fused epilogue for the
// state format.  fp32 moments: lane-contiguous units, a wave updates 1024 consecutive elements
// in 4 rounds of 256 (lane l holds elements 256 r + 4 l .. + 3 of round r); int8 moments: 16
// consecutive elements per thread.  N K is a multiple of 16384, so whole waves (and the
// quads and 16-lane int8 blocks inside them) are either in range or out of it.
template <int WT, int ST, int OPT>
__global__ __launch_bounds__(256) void optimizer_kernel(const float* dW, int64_t n_elem, EpiArgs e) {
  if constexpr (ST == FORGE_S_Q8) {  // int8 moments: 16 consecutive elements per thread (see seg_epilogue)
    const int64_t seg = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (seg * 16 >= n_elem) return;  // n_elem % 64 == 0: the 4 lanes of an int8 block leave together
    float gr[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 x = ld16(dW + seg * 16 + 4 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) gr[4 * q + c] = __uint_as_float(x[c]);
    }
    step_segment16<OPT, WT, ST>(gr, (uint32_t)(seg * 16), e);
    return;
  }
  const int64_t base = (((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6) * 1024;
  if (base >= n_elem) return;
  const int lane = (int)(threadIdx.x & 63);
  uint32_t i[4];
  UnitIn x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    i[r] = (uint32_t)(base + 256 * r + 4 * lane);
    unit_load<OPT, WT, ST>(x[r], i[r], e);
  }
  uint64_t w[4] = {0ull, 0ull, 0ull, 0ull};
  if (WT == FORGE_W_BF16 && e.sr) sr_words4(i, e, w);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x4 q = ld16(dW + i[r]);
    const float gr[4] = {__uint_as_float(q[0]), __uint_as_float(q[1]), __uint_as_float(q[2]), __uint_as_float(q[3])};
    unit_apply<OPT, WT, ST>(gr, i[r], x[r], w[r], e);
  }
}

// dX[T, K] = dY[T, N] . W[N, K], bf16 in, fp32 accumulate, bf16 (nearest-even) out.
// 256-token x 128-column tiles, the reduction over N in 32-wide slabs fed by LDS DMA
// (forge_mainloop2.h, dgrad section); two workgroups per CU.
static_assert(ml2::DgradPipe::SMEM <= kSmem2, "dgrad stages fit the shared buffer size");
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void dgrad_kernel2(const uint16_t* dY, const uint16_t* W,
                                                                     uint16_t* dX, int64_t T, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  const int nbT = (int)((T + ml2::BM - 1) / ml2::BM), nbK = (int)(K / ml2::BN);
  int tb, kb;
  tile_coords_at((int)blockIdx.x, nbT, nbK, tb, kb);
  const int64_t t0 = (int64_t)tb * ml2::BM;
  const int k0 = kb * ml2::BN;
  ml2::floatx4 acc[8][4];
  ml2::dgrad_contract(acc, smem, dY, W, T, N, K, t0, k0);
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    ml2::stage_acc_half(st, acc, 1.0f, half);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int row, kseg;
      seg_pos(s, row, kseg);
      const int64_t t = t0 + half * ml2::EPI_ROWS + row;
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
    __syncthreads();
  }
}

// dX tiles of 256 tokens x 256 columns, one workgroup of 8 waves per CU (forge_mainloop2.h, wide
// dgrad tiles): both 128-column halves share the dY slab and 4 slabs fit in LDS.  Each half
// stages its accumulators through its own LDS buffer and stores bf16 rows as dgrad_kernel2 does.
constexpr int kSmemDW =
    ml2::DgradWidePipe::SMEM > 2 * ml2::EPI_BYTES ? ml2::DgradWidePipe::SMEM : 2 * ml2::EPI_BYTES;
static_assert(kSmemDW <= 160 * 1024, "wide dgrad tiles fit the CU's LDS");

__global__ __launch_bounds__(2 * ml2::THREADS, 1) void dgrad_kernel2w(const uint16_t* dY, const uint16_t* W,
                                                                       uint16_t* dX, int64_t T, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemDW];
  const int nbT = (int)((T + ml2::BM - 1) / ml2::BM), nbK2 = (int)(K / (2 * ml2::BN));
  int tb, kb;
  tile_coords_at((int)blockIdx.x, nbT, nbK2, tb, kb);
  const int64_t t0 = (int64_t)tb * ml2::BM;
  const int kh = (int)(threadIdx.x >> 8);
  const int k0 = (2 * kb + kh) * ml2::BN;
  ml2::floatx4 acc[8][4];
  ml2::dgrad_wide_contract(acc, smem, dY, W, T, N, K, t0, 2 * kb * ml2::BN);
  float* st = reinterpret_cast<float*>(smem + kh * ml2::EPI_BYTES);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    ml2::stage_acc_half(st, acc, 1.0f, half);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int row, kseg;
      seg_pos(s, row, kseg);
      const int64_t t = t0 + half * ml2::EPI_ROWS + row;
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
    __syncthreads();
  }
}

// ------------------------------------------------------------------ dispatch tables
using FusedFn = void (*)(GemmArgs, EpiArgs);
using OptFn = void (*)(const float*, int64_t, EpiArgs);

template <int WT, int ST>
static FusedFn fused8_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return fused_step_kernel8<WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return fused_step_kernel8<WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return fused_step_kernel8<WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return fused_step_kernel8<WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return fused_step_kernel8<WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return fused_step_kernel8<WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return fused_step_kernel8<WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return fused_step_kernel8<WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}

template <int WT, int ST>
static FusedFn fused2_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return fused_step_kernel2<WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return fused_step_kernel2<WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return fused_step_kernel2<WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return fused_step_kernel2<WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return fused_step_kernel2<WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return fused_step_kernel2<WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return fused_step_kernel2<WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return fused_step_kernel2<WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}

template <int IN, int WT, int ST>
static FusedFn fused_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return fused_step_kernel<IN, WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return fused_step_kernel<IN, WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return fused_step_kernel<IN, WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return fused_step_kernel<IN, WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return fused_step_kernel<IN, WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return fused_step_kernel<IN, WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return fused_step_kernel<IN, WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return fused_step_kernel<IN, WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}

template <int IN>
static FusedFn fused_for(int w, int s, int opt) {
  if (w == FORGE_W_BF16) return s == FORGE_S_F32 ? fused_for<IN, FORGE_W_BF16, FORGE_S_F32>(opt)
                                                 : fused_for<IN, FORGE_W_BF16, FORGE_S_Q8>(opt);
  return s == FORGE_S_F32 ? fused_for<IN, FORGE_W_F32, FORGE_S_F32>(opt) : fused_for<IN, FORGE_W_F32, FORGE_S_Q8>(opt);
}

template <int WT, int ST>
static FusedFn fused8w_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return fused_step_kernel8w<WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return fused_step_kernel8w<WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return fused_step_kernel8w<WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return fused_step_kernel8w<WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return fused_step_kernel8w<WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return fused_step_kernel8w<WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return fused_step_kernel8w<WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return fused_step_kernel8w<WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}
template <int WT, int ST>
static FusedFn fused2w_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return fused_step_kernel2w<WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return fused_step_kernel2w<WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return fused_step_kernel2w<WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return fused_step_kernel2w<WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return fused_step_kernel2w<WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return fused_step_kernel2w<WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return fused_step_kernel2w<WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return fused_step_kernel2w<WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}
template <int WT, int ST>
static OptFn opt_for(int opt) {
  switch (opt) {
    case FORGE_OPT_ADAMW: return optimizer_kernel<WT, ST, FORGE_OPT_ADAMW>;
    case FORGE_OPT_NADAM: return optimizer_kernel<WT, ST, FORGE_OPT_NADAM>;
    case FORGE_OPT_RADAM: return optimizer_kernel<WT, ST, FORGE_OPT_RADAM>;
    case FORGE_OPT_LION: return optimizer_kernel<WT, ST, FORGE_OPT_LION>;
    case FORGE_OPT_RMSPROP: return optimizer_kernel<WT, ST, FORGE_OPT_RMSPROP>;
    case FORGE_OPT_ADAGRAD: return optimizer_kernel<WT, ST, FORGE_OPT_ADAGRAD>;
    case FORGE_OPT_SGD: return optimizer_kernel<WT, ST, FORGE_OPT_SGD>;
    case FORGE_OPT_SGD_MOMENTUM: return optimizer_kernel<WT, ST, FORGE_OPT_SGD_MOMENTUM>;
  }
  return nullptr;
}

int launch_fused_step(int in_type, int w_type, int s_type, int opt, const GemmArgs& g, const EpiArgs& e,
                      void* stream) {
  FusedFn fn = nullptr;
  if (use_v2(in_type, g)) {
    FusedFn fw = nullptr;
    if (w_type == FORGE_W_BF16) {
      fn = s_type == FORGE_S_F32 ? fused2_for<FORGE_W_BF16, FORGE_S_F32>(opt) : fused2_for<FORGE_W_BF16, FORGE_S_Q8>(opt);
      fw = s_type == FORGE_S_F32 ? fused2w_for<FORGE_W_BF16, FORGE_S_F32>(opt) : fused2w_for<FORGE_W_BF16, FORGE_S_Q8>(opt);
    } else {
      fn = s_type == FORGE_S_F32 ? fused2_for<FORGE_W_F32, FORGE_S_F32>(opt) : fused2_for<FORGE_W_F32, FORGE_S_Q8>(opt);
      fw = s_type == FORGE_S_F32 ? fused2w_for<FORGE_W_F32, FORGE_S_F32>(opt) : fused2w_for<FORGE_W_F32, FORGE_S_Q8>(opt);
    }
    if (!fn || !fw) return (int)hipErrorInvalidValue;
    GemmArgs g2 = g;
    g2.kb_base = 0;
    g2.nbk = (int)(g.K / ml2::BN);
    // wide tiles first; the columns they leave go to the 256 x 128 path in a second launch
    const int kw = plan_wide(g);
    if (kw > 0) {
      GemmArgs gw = g;
      gw.kb_base = 0;
      gw.nbk = 2 * kw;
      const unsigned gridw = (unsigned)((g.N / ml2::BM) * kw);
      hipLaunchKernelGGL(fw, dim3(gridw), dim3(2 * ml2::THREADS), 0, (hipStream_t)stream, gw, e);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return (int)err;
      g2.kb_base = 2 * kw;
      g2.nbk -= 2 * kw;
      if (g2.nbk == 0) return (int)hipSuccess;
    }
    const unsigned grid2 = plan_split(g2);
    hipLaunchKernelGGL(fn, dim3(grid2), dim3(ml2::THREADS), 0, (hipStream_t)stream, g2, e);
    return (int)hipGetLastError();
  }
  if (use_v8(in_type, g)) {
    FusedFn fw = nullptr;
    if (w_type == FORGE_W_BF16) {
      fn = s_type == FORGE_S_F32 ? fused8_for<FORGE_W_BF16, FORGE_S_F32>(opt) : fused8_for<FORGE_W_BF16, FORGE_S_Q8>(opt);
      fw = s_type == FORGE_S_F32 ? fused8w_for<FORGE_W_BF16, FORGE_S_F32>(opt) : fused8w_for<FORGE_W_BF16, FORGE_S_Q8>(opt);
    } else {
      fn = s_type == FORGE_S_F32 ? fused8_for<FORGE_W_F32, FORGE_S_F32>(opt) : fused8_for<FORGE_W_F32, FORGE_S_Q8>(opt);
      fw = s_type == FORGE_S_F32 ? fused8w_for<FORGE_W_F32, FORGE_S_F32>(opt) : fused8w_for<FORGE_W_F32, FORGE_S_Q8>(opt);
    }
    if (!fn || !fw) return (int)hipErrorInvalidValue;
    GemmArgs g8 = g;
    g8.kb_base = 0;
    g8.nbk = (int)(g.K / ml2::BN);
    // wide tiles first (same rule as for bf16 inputs); the rest on 256 x 128 tiles
    const int kw = plan_wide(g);
    if (kw > 0) {
      GemmArgs gw = g;
      gw.kb_base = 0;
      gw.nbk = 2 * kw;
      const unsigned gridw = (unsigned)((g.N / ml2::BM) * kw);
      hipLaunchKernelGGL(fw, dim3(gridw), dim3(2 * ml2::THREADS), 0, (hipStream_t)stream, gw, e);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return (int)err;
      g8.kb_base = 2 * kw;
      g8.nbk -= 2 * kw;
      if (g8.nbk == 0) return (int)hipSuccess;
    }
    const unsigned grid8 = (unsigned)((g.N / ml2::BM) * g8.nbk);
    hipLaunchKernelGGL(fn, dim3(grid8), dim3(ml2::THREADS), 0, (hipStream_t)stream, g8, e);
    return (int)hipGetLastError();
  }
  if (in_type == FORGE_IN_BF16) fn = fused_for<FORGE_IN_BF16>(w_type, s_type, opt);
  else if (in_type == FORGE_IN_F32) fn = fused_for<FORGE_IN_F32>(w_type, s_type, opt);
  else if (in_type == FORGE_IN_FP8) fn = fused_for<FORGE_IN_FP8>(w_type, s_type, opt);
  if (!fn) return (int)hipErrorInvalidValue;
  const unsigned grid = (unsigned)((g.N / kBM) * (g.K / kBN));
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, g, e);
  return (int)hipGetLastError();
}

int launch_wgrad_gemm(int in_type, const GemmArgs& g, float* dW, void* stream) {
  if (use_v2(in_type, g)) {
    GemmArgs g2 = g;
    g2.kb_base = 0;
    g2.nbk = (int)(g.K / ml2::BN);
    const unsigned grid2 = plan_split(g2);
    hipLaunchKernelGGL(wgrad_gemm_kernel2, dim3(grid2), dim3(ml2::THREADS), 0, (hipStream_t)stream, g2, dW);
    return (int)hipGetLastError();
  }
  if (use_v8(in_type, g)) {
    const unsigned grid8 = (unsigned)((g.N / ml2::BM) * (g.K / ml2::BN));
    hipLaunchKernelGGL(wgrad_gemm_kernel8, dim3(grid8), dim3(ml2::THREADS), 0, (hipStream_t)stream, g, dW);
    return (int)hipGetLastError();
  }
  const unsigned grid = (unsigned)((g.N / kBM) * (g.K / kBN));
  if (in_type == FORGE_IN_BF16)
    hipLaunchKernelGGL(wgrad_gemm_kernel<FORGE_IN_BF16>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, g, dW);
  else if (in_type == FORGE_IN_F32)
    hipLaunchKernelGGL(wgrad_gemm_kernel<FORGE_IN_F32>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, g, dW);
  else if (in_type == FORGE_IN_FP8)
    hipLaunchKernelGGL(wgrad_gemm_kernel<FORGE_IN_FP8>, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, g, dW);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int launch_optimizer(int w_type, int s_type, int opt, const float* dW, int64_t n_elem, const EpiArgs& e,
                     void* stream) {
  OptFn fn;
  if (w_type == FORGE_W_BF16)
    fn = s_type == FORGE_S_F32 ? opt_for<FORGE_W_BF16, FORGE_S_F32>(opt) : opt_for<FORGE_W_BF16, FORGE_S_Q8>(opt);
  else
    fn = s_type == FORGE_S_F32 ? opt_for<FORGE_W_F32, FORGE_S_F32>(opt) : opt_for<FORGE_W_F32, FORGE_S_Q8>(opt);
  if (!fn) return (int)hipErrorInvalidValue;
  const unsigned grid = (unsigned)((n_elem + 4095) / 4096);   // 4 waves of 1024 elements a block
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, (hipStream_t)stream, dW, n_elem, e);
  return (int)hipGetLastError();
}

// Wide dgrad tiles need K % 256 == 0 and at least one tile per CU.
static bool use_dgrad_wide(int64_t T, int64_t K) {
  const int64_t tiles = ((T + ml2::BM - 1) / ml2::BM) * (K / (2 * ml2::BN));
  return K % (2 * ml2::BN) == 0 && tiles >= slots_on_current_device() / 2;
}

int launch_dgrad(const void* dY, const void* W, void* dX, int64_t T, int64_t N, int64_t K, void* stream) {
  if (use_dgrad_wide(T, K)) {
    const unsigned gridw = (unsigned)(((T + ml2::BM - 1) / ml2::BM) * (K / (2 * ml2::BN)));
    hipLaunchKernelGGL(dgrad_kernel2w, dim3(gridw), dim3(2 * ml2::THREADS), 0, (hipStream_t)stream,
                       static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(W), static_cast<uint16_t*>(dX),
                       T, N, K);
    return (int)hipGetLastError();
  }
  const unsigned grid = (unsigned)(((T + ml2::BM - 1) / ml2::BM) * (K / ml2::BN));
  hipLaunchKernelGGL(dgrad_kernel2, dim3(grid), dim3(ml2::THREADS), 0, (hipStream_t)stream,
                     static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(W), static_cast<uint16_t*>(dX), T,
                     N, K);
  return (int)hipGetLastError();
}

}  // namespace forge
