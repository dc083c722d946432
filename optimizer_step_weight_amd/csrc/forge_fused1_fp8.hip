// forge_fused1_fp8.hip -- fused step kernels for fp8 inputs, register-staged 128 x 128 tiles.
#include "forge_fused1.h"

namespace forge {
template FusedFn select_fused1<FORGE_IN_FP8>(int, int, int, int);
}  // namespace forge
