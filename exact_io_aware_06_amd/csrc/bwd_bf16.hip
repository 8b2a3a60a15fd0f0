// Attention backward, bfloat16: the preprocess kernel, the dispatch, and
// the dK/dV and dQ instantiations without a causal or window edge (the
// others are in bwd_bf16_masked.hip; two files so that they build in
// parallel). The build compiles both with the compiler's iterative-maxocc
// scheduling strategy: on the dK/dV kernel it removes most MFMAs that wait
// directly on their LDS read (headline backward 1.91 -> 1.76 ms).

#include "bwd_bf16_kernel.h"

namespace attn {
namespace {

// ------------------------------------------------------------- preprocess
// LPR lanes per query row, 8 elements (16 bytes) of O and dO per lane.
template <int LPR>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int kRows = 256 / LPR;  // rows per workgroup
  const int sub = threadIdx.x % LPR;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  const int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / LPR;
  const bool ok = row < rows;
  const int64_t rr = ok ? row : rows - 1;
  const int i = (int)(rr % p.Nq);
  const int h = (int)((rr / p.Nq) % p.H);
  const int b = (int)(rr / ((int64_t)p.Nq * p.H));
  const __bf16* orow = static_cast<const __bf16*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_sn;
  const __bf16* drow = static_cast<const __bf16*>(p.do_) + b * p.do_sb + h * p.do_sh + (int64_t)i * p.do_sn;
  const bf16x8 ov = *reinterpret_cast<const bf16x8*>(orow + 8 * sub);
  const bf16x8 dv = *reinterpret_cast<const bf16x8*>(drow + 8 * sub);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc = __builtin_fmaf((float)ov[c], (float)dv[c], acc);
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && sub == 0) {
    p.dsum[row] = acc;
    const float l = p.lse[b * p.l_sb + h * p.l_sh + i];
    p.lse2[row] = (l == -INFINITY) ? -INFINITY : -l * kLog2e;
  }
}

// Zero fill of a strided [B, H, N, d] bf16 tensor: d / 8 lanes per row, one
// 16-byte store each, grid-stride over all rows.
__global__ __launch_bounds__(256) void zero_rows_kernel(__bf16* data, int64_t rows, int H, int N,
                                                        int d8, int64_t sb, int64_t sh, int64_t sn) {
  const int64_t total = rows * d8;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
    const int64_t r = t / d8;
    const int c = (int)(t % d8);
    const int n = (int)(r % N);
    const int h = (int)((r / N) % H);
    const int64_t b = r / ((int64_t)N * H);
    *reinterpret_cast<uint4*>(data + b * sb + h * sh + n * sn + 8 * c) = uint4{0, 0, 0, 0};
  }
}

}  // namespace

int launch_zero_bf16(void* data, int64_t B, int64_t H, int64_t N, int d, int64_t sb, int64_t sh,
                     int64_t sn, void* stream) {
  const int64_t rows = B * H * N;
  if (rows == 0) return (int)hipSuccess;
  const int64_t want = (rows * (d / 8) + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(zero_rows_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<__bf16*>(data), rows, (int)H, (int)N, d / 8, sb, sh, sn);
  return (int)hipGetLastError();
}

hipError_t launch_bwd_unmasked(const BwdParams& p, int d, hipStream_t s) {
  const bool bias = p.bias != nullptr;
  if (d == 128)
    return bias ? launch_bwd_d<128, false, true, false>(p, s) : launch_bwd_d<128, false, false, false>(p, s);
  if (d == 64)
    return bias ? launch_bwd_d<64, false, true, false>(p, s) : launch_bwd_d<64, false, false, false>(p, s);
  return hipErrorInvalidValue;
}

int launch_bwd_bf16(const BwdParams& p, int d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d != 64 && d != 128) return (int)hipErrorInvalidValue;
  const int64_t rows = (int64_t)p.B * p.H * p.Nq;
  if (rows > 0) {
    if (d == 128) hipLaunchKernelGGL(bwd_pre_kernel<16>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bwd_pre_kernel<8>, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)(p.causal || p.local ? launch_bwd_masked(p, d, s) : launch_bwd_unmasked(p, d, s));
}

}  // namespace attn
