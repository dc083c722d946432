// forge_fused2_f32.hip -- fused step kernels for bf16 inputs, fp32 moments.
#include "forge_fused2.h"

namespace forge {
template FusedFn select_fused2<FORGE_S_F32>(int, int, int);
}  // namespace forge
