// forge_kernels.hip -- launchers of the fused and the unfused paths, and the unfused and dgrad
// kernels.  The fused kernels live in forge_fused{1,2,8}.h, each instantiated in its own
// translation units; the shared epilogue in forge_epilogue.h.
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
//     (forge_mainloop.h), 64 x 64 for fp32 layers with fewer 128 x 128 tiles than CUs.
// The element-wise update of a 16-element segment (forge_device.h) is shared by all of them.
//
// Unfused baseline (Technical Summary section 1 "The Problem"): the same contraction writes
// the fp32 gradient to HBM, and a separate element-wise kernel reads it back and applies the
// same update code.
//
// dgrad: dX = dY W on the LDS-DMA path (256-token x 256-column tiles in one 8-wave workgroup
// per CU where K % 256 == 0 and they fill the CUs, else 256 x 128), run before the step so
// that it sees the old weight (Technical Summary section 5, limitations).  The same dgrad and
// step in one launch: forge_backward.hip.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "forge_dgrad.h"

namespace forge {

template <int IN, int S>
__global__ __launch_bounds__(kThreads, S == 128 ? 2 : 4) void wgrad_gemm_kernel(GemmArgs g, float* dW) {
  using TL = SmallTile<S>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[TL::SMEM];
  const int nbN = (int)(g.N / S), nbK = (int)(g.K / S);
  int nb, kb;
  tile_coords(nbN, nbK, nb, kb);
  const int n0 = nb * S, k0 = kb * S;

  floatx4 acc[TL::NB][TL::NB];
  contract_tile<IN, S>(acc, smem, g, n0, k0);

  float* st = reinterpret_cast<float*>(smem);
  stage_acc<S>(st, acc, input_scale<IN>(g));
  __syncthreads();
#pragma unroll
  for (int s = 0; s < TL::SEGS; ++s) {
    int row, col;
    small_seg<S>(s, row, col);
    const float* p = st + row * kEpiLd + col;
    float* d = dW + (int64_t)(n0 + row) * g.K + k0 + col;
#pragma unroll
    for (int q = 0; q < 4; ++q) st16(d + 4 * q, *reinterpret_cast<const u32x4*>(p + 4 * q));
  }
}

__global__ __launch_bounds__(ml2::THREADS, kOcc2) void wgrad_gemm_kernel2(GemmArgs g, float* dW) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  float* st = reinterpret_cast<float*>(smem);
  const int b = (int)blockIdx.x;
  int n0, k0;
  if (b < g.nfull) {
    plan::full_tile(g, b, n0, k0);
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
    plan::half_tile(g, b - g.nfull, n0, k0);
    ml2::floatx4 acc[4][4];
    ml2::contract<Pipe2H>(acc, smem, g, n0, k0);
    ml2::stage_acc_all(st, acc, 1.0f);
    __syncthreads();
    store_staged(st, dW, g.K, n0, k0);
  }
}

__global__ __launch_bounds__(ml2::THREADS, kOcc2) void wgrad_gemm_kernel8(GemmArgs g, float* dW) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  int n0, k0;
  plan::tile8(g, (int)blockIdx.x, n0, k0);
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
int slots_on_current_device() {
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

// Element-wise rule over a materialised gradient, in the layout of the fused epilogue for the
// state format.  fp32 moments: lane-contiguous units, a wave updates 1024 consecutive elements
// in 4 rounds of 256 (lane l holds elements 256 r + 4 l .. + 3 of round r); int8 moments: 16
// consecutive elements per thread.  N K is a multiple of 16384, so whole waves (and the
// quads and 16-lane int8 blocks inside them) are either in range or out of it.
template <int WT, int ST, int OPT>
__global__ __launch_bounds__(256) void optimizer_kernel(const float* dW, int64_t n_elem, EpiArgs e) {
  if constexpr (ST != FORGE_S_F32) {  // int8 moments: 16 consecutive elements per thread (see seg_epilogue)
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

// dX[T, K] = dY[T, N] . W[N, K] on 256-token x 128-column tiles (forge_dgrad.h), two
// workgroups per CU.
static_assert(ml2::DgradPipe::SMEM <= kSmem2, "dgrad stages fit the shared buffer size");
__global__ __launch_bounds__(ml2::THREADS, kOcc2) void dgrad_kernel2(const uint16_t* dY, const uint16_t* W,
                                                                     uint16_t* dX, int64_t T, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem2];
  const int nbT = (int)((T + ml2::BM - 1) / ml2::BM), nbK = (int)(K / ml2::BN);
  int tb, kb;
  tile_coords_at((int)blockIdx.x, nbT, nbK, tb, kb);
  dgrad_tile(dY, W, dX, T, N, K, (int64_t)tb * ml2::BM, kb * ml2::BN, smem, [] {});
}

// dX tiles of 256 tokens x 256 columns, one workgroup of 8 waves per CU (forge_dgrad.h).
constexpr int kSmemDW =
    ml2::DgradWidePipe::SMEM > 2 * ml2::EPI_BYTES ? ml2::DgradWidePipe::SMEM : 2 * ml2::EPI_BYTES;
static_assert(kSmemDW <= 160 * 1024, "wide dgrad tiles fit the CU's LDS");

__global__ __launch_bounds__(2 * ml2::THREADS, 1) void dgrad_kernel2w(const uint16_t* dY, const uint16_t* W,
                                                                       uint16_t* dX, int64_t T, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemDW];
  const int nbT = (int)((T + ml2::BM - 1) / ml2::BM), nbK2 = (int)(K / (2 * ml2::BN));
  int tb, kb;
  tile_coords_at((int)blockIdx.x, nbT, nbK2, tb, kb);
  dgrad_tile_wide(dY, W, dX, T, N, K, (int64_t)tb * ml2::BM, 2 * kb * ml2::BN, smem);
}

// ------------------------------------------------------------------ dispatch tables
using OptFn = void (*)(const float*, int64_t, EpiArgs);

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

static FusedFn fused2_for(int s_type, int wide, int w_type, int opt) {
  return s_type == FORGE_S_F32  ? select_fused2<FORGE_S_F32>(wide, w_type, opt)
         : s_type == FORGE_S_Q8 ? select_fused2<FORGE_S_Q8>(wide, w_type, opt)
                                : select_fused2<FORGE_S_Q8D>(wide, w_type, opt);
}
static FusedFn fused8_for(int s_type, int wide, int w_type, int opt) {
  return s_type == FORGE_S_F32  ? select_fused8<FORGE_S_F32>(wide, w_type, opt)
         : s_type == FORGE_S_Q8 ? select_fused8<FORGE_S_Q8>(wide, w_type, opt)
                                : select_fused8<FORGE_S_Q8D>(wide, w_type, opt);
}

int launch_fused_step(int in_type, int w_type, int s_type, int opt, const GemmArgs& g, const EpiArgs& e,
                      void* stream) {
  plan::Launch L[2];
  const int n = plan::plan_launches(in_type, g, slots_on_current_device() / 2, 1, L);
  for (int i = 0; i < n; ++i) {
    FusedFn fn = nullptr;
    unsigned threads = ml2::THREADS;
    if (L[i].kind == plan::LAUNCH_WIDE) {
      fn = in_type == FORGE_IN_BF16 ? fused2_for(s_type, 1, w_type, opt) : fused8_for(s_type, 1, w_type, opt);
      threads = 2 * ml2::THREADS;
    } else if (L[i].kind == plan::LAUNCH_V2) {
      fn = fused2_for(s_type, 0, w_type, opt);
    } else if (L[i].kind == plan::LAUNCH_V8) {
      fn = fused8_for(s_type, 0, w_type, opt);
    } else {
      const int tile = L[i].tile;
      if (in_type == FORGE_IN_BF16) fn = select_fused1<FORGE_IN_BF16>(w_type, s_type, opt, tile);
      else if (in_type == FORGE_IN_F32) fn = select_fused1<FORGE_IN_F32>(w_type, s_type, opt, tile);
      else if (in_type == FORGE_IN_FP8) fn = select_fused1<FORGE_IN_FP8>(w_type, s_type, opt, tile);
      threads = kThreads;
    }
    if (!fn) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(L[i].grid), dim3(threads), 0, (hipStream_t)stream, L[i].g, e);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return (int)err;
  }
  return (int)hipSuccess;
}

int launch_wgrad_gemm(int in_type, const GemmArgs& g, float* dW, void* stream) {
  plan::Launch L[2];
  const int n = plan::plan_launches(in_type, g, slots_on_current_device() / 2, 0, L);
  for (int i = 0; i < n; ++i) {
    const GemmArgs& gl = L[i].g;
    const dim3 grid(L[i].grid);
    if (L[i].kind == plan::LAUNCH_V2)
      hipLaunchKernelGGL(wgrad_gemm_kernel2, grid, dim3(ml2::THREADS), 0, (hipStream_t)stream, gl, dW);
    else if (L[i].kind == plan::LAUNCH_V8)
      hipLaunchKernelGGL(wgrad_gemm_kernel8, grid, dim3(ml2::THREADS), 0, (hipStream_t)stream, gl, dW);
    else if (L[i].kind == plan::LAUNCH_SMALL && in_type == FORGE_IN_BF16 && L[i].tile == 128)
      hipLaunchKernelGGL((wgrad_gemm_kernel<FORGE_IN_BF16, 128>), grid, dim3(kThreads), 0, (hipStream_t)stream, gl, dW);
    else if (L[i].kind == plan::LAUNCH_SMALL && in_type == FORGE_IN_F32 && L[i].tile == 128)
      hipLaunchKernelGGL((wgrad_gemm_kernel<FORGE_IN_F32, 128>), grid, dim3(kThreads), 0, (hipStream_t)stream, gl, dW);
    else if (L[i].kind == plan::LAUNCH_SMALL && in_type == FORGE_IN_F32 && L[i].tile == 64)
      hipLaunchKernelGGL((wgrad_gemm_kernel<FORGE_IN_F32, 64>), grid, dim3(kThreads), 0, (hipStream_t)stream, gl, dW);
    else if (L[i].kind == plan::LAUNCH_SMALL && in_type == FORGE_IN_FP8 && L[i].tile == 128)
      hipLaunchKernelGGL((wgrad_gemm_kernel<FORGE_IN_FP8, 128>), grid, dim3(kThreads), 0, (hipStream_t)stream, gl, dW);
    else
      return (int)hipErrorInvalidValue;
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return (int)err;
  }
  return (int)hipSuccess;
}

int launch_optimizer(int w_type, int s_type, int opt, const float* dW, int64_t n_elem, const EpiArgs& e,
                     void* stream) {
  OptFn fn = nullptr;
  if (w_type == FORGE_W_BF16)
    fn = s_type == FORGE_S_F32 ? opt_for<FORGE_W_BF16, FORGE_S_F32>(opt)
         : s_type == FORGE_S_Q8 ? opt_for<FORGE_W_BF16, FORGE_S_Q8>(opt)
                                : opt_for<FORGE_W_BF16, FORGE_S_Q8D>(opt);
  else
    fn = s_type == FORGE_S_F32 ? opt_for<FORGE_W_F32, FORGE_S_F32>(opt)
         : s_type == FORGE_S_Q8 ? opt_for<FORGE_W_F32, FORGE_S_Q8>(opt)
                                : opt_for<FORGE_W_F32, FORGE_S_Q8D>(opt);
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

