// forge_fused8_f32.hip -- fused step kernels for fp8 inputs, fp32 moments.
#include "forge_fused8.h"

namespace forge {
template FusedFn select_fused8<FORGE_S_F32>(int, int, int);
}  // namespace forge
