// forge_fused1_f32.hip -- fused step kernels for fp32 inputs, register-staged 128 x 128 and
// 64 x 64 tiles.
#include "forge_fused1.h"

namespace forge {
template FusedFn select_fused1<FORGE_IN_F32>(int, int, int, int);
}  // namespace forge
