// bf16 forward over packed variable-length sequences (with or without a
// window); no bias, no key split.

#include "fwd_bf16_kernel.h"

namespace attn {

hipError_t launch_bf16_varlen(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  if (p.local) return launch_family<false, true, true>(p, tm, d, waves, s);
  return launch_family<false, false, true>(p, tm, d, waves, s);
}

}  // namespace attn
