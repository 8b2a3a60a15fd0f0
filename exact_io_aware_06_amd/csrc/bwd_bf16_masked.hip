// Attention backward, bfloat16: the dK/dV and dQ instantiations with a
// causal or window edge (the unmasked ones, the preprocess and the dispatch
// are in bwd_bf16.hip).

#include "bwd_bf16_kernel.h"

namespace attn {

template <int D>
static hipError_t launch_masked_d(const BwdParams& p, hipStream_t s) {
  const bool bias = p.bias != nullptr;
  if (p.local)
    return bias ? launch_bwd_d<D, true, true, true>(p, s) : launch_bwd_d<D, true, false, true>(p, s);
  return bias ? launch_bwd_d<D, true, true, false>(p, s) : launch_bwd_d<D, true, false, false>(p, s);
}

hipError_t launch_bwd_masked(const BwdParams& p, int d, hipStream_t s) {
  if (d == 128) return launch_masked_d<128>(p, s);
  if (d == 64) return launch_masked_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
