// forge_fused8_q8.hip -- fused step kernels for fp8 inputs, int8 block-64 moments.
#include "forge_fused8.h"

namespace forge {
template FusedFn select_fused8<FORGE_S_Q8>(int, int, int);
}  // namespace forge
