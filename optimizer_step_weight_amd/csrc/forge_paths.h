// forge_paths.h -- the fused kernels' per-path selectors, each explicitly instantiated in its
// own translation unit (so that the paths compile in parallel).
#pragma once

#include "forge_internal.h"

namespace forge {

using FusedFn = void (*)(GemmArgs, EpiArgs);

#define FORGE_FOR_EACH_OPT(X)                                                                               \
  X(FORGE_OPT_ADAMW) X(FORGE_OPT_NADAM) X(FORGE_OPT_RADAM) X(FORGE_OPT_LION) X(FORGE_OPT_RMSPROP)          \
  X(FORGE_OPT_ADAGRAD) X(FORGE_OPT_SGD) X(FORGE_OPT_SGD_MOMENTUM)

// bf16 inputs, LDS-DMA path: wide = 1 selects the 256 x 256 kernel, 0 the 256 x 128 one.
template <int ST>
FusedFn select_fused2(int wide, int w_type, int opt);
// fp8 inputs, LDS-DMA path: same tiles.
template <int ST>
FusedFn select_fused8(int wide, int w_type, int opt);
// register-staged path for input format IN on tiles of side `tile` (128, or 64 for fp32).
template <int IN>
FusedFn select_fused1(int w_type, int s_type, int opt, int tile);

extern template FusedFn select_fused2<FORGE_S_F32>(int, int, int);
extern template FusedFn select_fused2<FORGE_S_Q8>(int, int, int);
extern template FusedFn select_fused2<FORGE_S_Q8D>(int, int, int);
extern template FusedFn select_fused8<FORGE_S_F32>(int, int, int);
extern template FusedFn select_fused8<FORGE_S_Q8>(int, int, int);
extern template FusedFn select_fused8<FORGE_S_Q8D>(int, int, int);
extern template FusedFn select_fused1<FORGE_IN_F32>(int, int, int, int);
extern template FusedFn select_fused1<FORGE_IN_BF16>(int, int, int, int);
extern template FusedFn select_fused1<FORGE_IN_FP8>(int, int, int, int);

}  // namespace forge
