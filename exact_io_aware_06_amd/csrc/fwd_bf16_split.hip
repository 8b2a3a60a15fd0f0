// bf16 forward, split-key instantiations (flash-decoding partials).

#include "fwd_bf16_kernel.h"

namespace attn {

hipError_t launch_bf16_split(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  return launch_family<true, false>(p, tm, d, waves, s);
}

}  // namespace attn
