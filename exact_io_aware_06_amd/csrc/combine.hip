// Merge of split-over-keys partial results (flash-decoding), gfx950.
//
// A split launch of the forward leaves, for every query row and every split
// s of the keys, the split's own normalised output O_s (fp32) and its
// log-sum-exp L_s (natural log, -inf when the split saw no key of that row).
// The exact result over all keys follows from the merge identity of the
// blockwise softmax ("Understanding FlashAttention Pt 1: Personal Notes",
// section 2.4; "FlashAttention: Mathematical Foundations...", section 7,
// flash-decoding): with M = max_s L_s and w_s = exp(L_s - M),
//
//     O = sum_s w_s O_s / sum_s w_s,      LSE = M + log(sum_s w_s).
//
// A row whose splits are all empty (M = -inf) gets O = 0 and LSE = -inf,
// the same rule as the forward.
//
// One wavefront per row: the lanes first share the split log-sum-exps (64
// splits per pass), then each lane accumulates d/64 adjacent columns of the
// output over the splits, so every read of a split's row is one contiguous
// d * 4-byte segment.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kRowsPerBlock = 4;  // wavefronts (rows) per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// CPL = output columns per lane (d / 64)
template <int CPL>
__global__ __launch_bounds__(64 * kRowsPerBlock) void combine_bf16_kernel(FwdParams p) {
  constexpr int D = 64 * CPL;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % p.Nq);
  const int h = (int)((row / p.Nq) % p.H);
  const int b = (int)(row / ((int64_t)p.Nq * p.H));
  const int ns = p.n_split;
  // partial (s, row) sits at s * rows + row
  const float* lse_s = p.part_lse + row;
  const float* o_s = p.part_o + row * D + CPL * lane;

  float m = -INFINITY;
  for (int s = lane; s < ns; s += 64) m = fmaxf(m, lse_s[(int64_t)s * rows]);
  m = wave_max(m);

  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    const float m2 = m * kLog2e;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      // lane t holds the weight of split s0 + t
      float w = 0.f;
      if (s0 + lane < ns) w = __builtin_amdgcn_exp2f(__builtin_fmaf(lse_s[(int64_t)(s0 + lane) * rows], kLog2e, -m2));
      wsum += w;
      const int cnt = min(64, ns - s0);
      for (int t = 0; t < cnt; ++t) {
        const float wt = __shfl(w, t, 64);
        const float* src = o_s + (int64_t)(s0 + t) * rows * D;
        if constexpr (CPL == 2) {
          const float2 x = *reinterpret_cast<const float2*>(src);
          acc[0] = __builtin_fmaf(wt, x.x, acc[0]);
          acc[1] = __builtin_fmaf(wt, x.y, acc[1]);
        } else {
          acc[0] = __builtin_fmaf(wt, src[0], acc[0]);
        }
      }
    }
    wsum = wave_sum(wsum);
  }
  // w_s = 1 for the split holding the maximum, so wsum >= 1 when m is finite
  const float inv = (m != -INFINITY) ? 1.f / wsum : 0.f;
  __bf16* orow = static_cast<__bf16*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_sn + CPL * lane;
#pragma unroll
  for (int c = 0; c < CPL; ++c) orow[c] = (__bf16)(acc[c] * inv);
  if (lane == 0) {
    float* lrow = p.lse + b * p.l_sb + h * p.l_sh;
    lrow[i] = (m != -INFINITY) ? m + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
  }
}

}  // namespace

int launch_combine_bf16(const FwdParams& p, int d, void* stream) {
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid == 0) return (int)hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 128)
    hipLaunchKernelGGL(combine_bf16_kernel<2>, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(combine_bf16_kernel<1>, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0, s, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace attn
