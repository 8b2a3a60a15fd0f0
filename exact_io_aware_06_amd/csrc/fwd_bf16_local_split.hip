// bf16 forward, sliding-window instantiations with a key split.

#include "fwd_bf16_kernel.h"

namespace attn {

hipError_t launch_bf16_local_split(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  return launch_family<true, true>(p, tm, d, waves, s);
}

}  // namespace attn
