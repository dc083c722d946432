// forge_fused2_q8d.hip -- fused step kernels for bf16 inputs, 8-bit block-64 moments in the
// dynamic map.
#include "forge_fused2.h"

namespace forge {
template FusedFn select_fused2<FORGE_S_Q8D>(int, int, int);
}  // namespace forge
