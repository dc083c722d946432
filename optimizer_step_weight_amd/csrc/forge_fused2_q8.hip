// forge_fused2_q8.hip -- fused step kernels for bf16 inputs, int8 block-64 moments.
#include "forge_fused2.h"

namespace forge {
template FusedFn select_fused2<FORGE_S_Q8>(int, int, int);
}  // namespace forge
