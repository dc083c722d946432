// forge_internal.h -- structures shared by the host entry points and the kernels.
#pragma once

#include <stdint.h>

namespace forge {

enum : int {
  FORGE_OPT_ADAMW = 0,
  FORGE_OPT_NADAM = 1,
  FORGE_OPT_RADAM = 2,
  FORGE_OPT_LION = 3,
  FORGE_OPT_RMSPROP = 4,
  FORGE_OPT_ADAGRAD = 5,
  FORGE_OPT_SGD = 6,
  FORGE_OPT_SGD_MOMENTUM = 7,
};

// input element type of X and dY
enum : int { FORGE_IN_F32 = 0, FORGE_IN_BF16 = 1, FORGE_IN_FP8 = 2 };
// weight storage
enum : int { FORGE_W_F32 = 0, FORGE_W_BF16 = 1 };
// moment storage: fp32, or 8-bit codes with block-64 fp32 scales in the linear absmax map
// (Q8) or the dynamic map (Q8D)
enum : int { FORGE_S_F32 = 0, FORGE_S_Q8 = 1, FORGE_S_Q8D = 2 };

// Per-step scalars of a rule, computed on the host in fp64 and rounded to fp32.
struct OptScalars {
  float decay;  // 1 - lr*wd when weight decay is decoupled, else 1
  float l2;     // wd when weight decay is coupled (added to the gradient), else 0
  float c1, c2, c3;
  float b1, omb1, b2, omb2;
  float eps, lr;
  int32_t rect;  // RAdam: rectified branch this step
};

// Everything the optimizer epilogue needs.
struct EpiArgs {
  void* W;         // [N, K] fp32 or bf16
  void* m;         // [N, K] fp32 or int8 codes, or null
  void* v;         // [N, K] fp32 or uint8 codes, or null
  float* m_scale;  // [N*K/64] block absmax (int8 moments)
  float* v_scale;
  float* w_pre;    // optional fp32 copy of the weight before rounding
  uint64_t seed;
  uint64_t step;
  int32_t sr;      // bf16 weight: stochastic (1) or nearest-even (0) rounding
  OptScalars s;
};

// The contraction dW = dY^T X.
struct GemmArgs {
  const void* X;   // [T, K]
  const void* dY;  // [T, N]
  const float* x_scale;   // fp8 per-tensor scales (device), else null
  const float* dy_scale;
  int64_t T, N, K;
  // LDS-DMA paths (set by the launcher): the launch covers the nbn 256-row blocks from nb_base
  // on and the nbk 128-column blocks from kb_base on; on the 256 x 128 path workgroups
  // [0, nfull) take 256 x 128 tiles of column blocks [0, kb_split) of that range and the rest
  // 128 x 128 tiles of column blocks [kb_split, nbk).
  int nfull = 0, kb_split = 0, kb_base = 0, nbk = 0, nb_base = 0, nbn = 0;
  // Wide launches on bf16 inputs (forge_plan.h, wide_item): the nfull 256 x 256 tiles cover
  // the nbn row blocks from nb_base on and the kb_split column blocks from kb_base on; the
  // 128 x 256 half-wide tiles cover the hn row blocks from h_nb on and the hk column blocks
  // from h_kb on, nfront of them dispatched before the wide tiles and the rest after.
  int nfront = 0, h_nb = 0, hn = 0, h_kb = 0, hk = 0;
};

// Launchers (defined in the .hip translation units).  Return a hipError_t as int.
int launch_fused_step(int in_type, int w_type, int s_type, int opt, const GemmArgs& g, const EpiArgs& e,
                      void* stream);
int launch_wgrad_gemm(int in_type, const GemmArgs& g, float* dW, void* stream);
int launch_optimizer(int w_type, int s_type, int opt, const float* dW, int64_t n_elem, const EpiArgs& e,
                     void* stream);
int launch_dgrad(const void* dY, const void* W, void* dX, int64_t T, int64_t N, int64_t K, void* stream);

// The backward step in one launch (forge_backward.hip): dX tiles and the fused step's tiles
// taken from work queues, the step's update of a column block after that block's dX tiles.
struct BackwardArgs {
  const uint16_t* W_old;  // W [N, K] bf16 as the dX tiles read it (the weight the step updates)
  uint16_t* dX;           // [T, K] bf16
  int* ctr;               // workspace words (forge_backward.hip)
  int nbT;                // 256-token blocks of dX
  int n_dgrad;            // dX tiles: nbT x (K / 128)
  int spin_limit;         // polls of a wait before it gives up
};
constexpr int kBackwardSpinLimit = 1 << 21;
// Workspace words for a weight of K columns.
int64_t backward_workspace_words(int64_t K);
// The allocation-free variant's counters: a static device array of this many words per device;
// backward_scratch() gives its address on the current device (resolved once per device).
constexpr int kBackwardScratchWords = 4096;
int backward_scratch(int** out);
int launch_backward_step(int s_type, int opt, const GemmArgs& g, const EpiArgs& e, const void* W_old, void* dX,
                         int* ctr, void* stream);
// Workgroup slots of the current device: two per CU.
int slots_on_current_device();

}  // namespace forge
