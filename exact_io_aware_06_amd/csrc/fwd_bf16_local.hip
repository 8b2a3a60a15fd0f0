// bf16 forward, sliding-window instantiations without a key split; the
// split ones are in fwd_bf16_local_split.hip.

#include "fwd_bf16_kernel.h"

namespace attn {

hipError_t launch_bf16_local_split(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s);

hipError_t launch_bf16_local(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  if (p.n_split > 1) return launch_bf16_local_split(p, tm, d, waves, s);
  return launch_family<false, true>(p, tm, d, waves, s);
}

}  // namespace attn
