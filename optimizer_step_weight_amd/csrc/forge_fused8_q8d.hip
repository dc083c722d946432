// forge_fused8_q8d.hip -- fused step kernels for fp8 e4m3 inputs, 8-bit block-64 moments in the
// dynamic map.
#include "forge_fused8.h"

namespace forge {
template FusedFn select_fused8<FORGE_S_Q8D>(int, int, int);
}  // namespace forge
