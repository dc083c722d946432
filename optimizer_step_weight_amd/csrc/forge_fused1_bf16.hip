// forge_fused1_bf16.hip -- fused step kernels for bf16 inputs, register-staged 128 x 128 tiles.
#include "forge_fused1.h"

namespace forge {
template FusedFn select_fused1<FORGE_IN_BF16>(int, int, int, int);
}  // namespace forge
