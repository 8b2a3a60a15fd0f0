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
// LPR lanes per query row, 8 elements (16 bytes) of O and dO per lane, kRep
// rows per lane (their loads issued together).
// GRID3: workgroup (x, h, b) takes kRep * kRows rows of head h of batch b
// from row x * kRep * kRows on (no per-lane division); else a flat grid over
// all B * H * Nq rows (for H or B beyond a grid dimension's 65535).
constexpr int kPreRep = 4;
template <int LPR, bool GRID3>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int kRows = 256 / LPR;  // rows per workgroup and repetition
  const int sub = threadIdx.x % LPR;
  int i[kPreRep], h[kPreRep], b[kPreRep];
  bool ok[kPreRep];
  int64_t row[kPreRep];
  bf16x8 ov[kPreRep], dv[kPreRep];
  float lv[kPreRep];
#pragma unroll
  for (int r = 0; r < kPreRep; ++r) {
    if constexpr (GRID3) {
      h[r] = blockIdx.y;
      b[r] = blockIdx.z;
      const int i0 = (blockIdx.x * kPreRep + r) * kRows + threadIdx.x / LPR;
      ok[r] = i0 < p.Nq;
      i[r] = ok[r] ? i0 : p.Nq - 1;
      row[r] = ((int64_t)b[r] * p.H + h[r]) * p.Nq + i[r];
    } else {
      const int64_t rows = (int64_t)p.B * p.H * p.Nq;
      row[r] = ((int64_t)blockIdx.x * kPreRep + r) * kRows + threadIdx.x / LPR;
      ok[r] = row[r] < rows;
      const int64_t rr = ok[r] ? row[r] : rows - 1;
      i[r] = (int)(rr % p.Nq);
      h[r] = (int)((rr / p.Nq) % p.H);
      b[r] = (int)(rr / ((int64_t)p.Nq * p.H));
    }
    const __bf16* orow = static_cast<const __bf16*>(p.o) + b[r] * p.o_sb + h[r] * p.o_sh + (int64_t)i[r] * p.o_sn;
    const __bf16* drow = static_cast<const __bf16*>(p.do_) + b[r] * p.do_sb + h[r] * p.do_sh + (int64_t)i[r] * p.do_sn;
    ov[r] = *reinterpret_cast<const bf16x8*>(orow + 8 * sub);
    dv[r] = *reinterpret_cast<const bf16x8*>(drow + 8 * sub);
    lv[r] = p.lse[b[r] * p.l_sb + h[r] * p.l_sh + i[r]];
  }
#pragma unroll
  for (int r = 0; r < kPreRep; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc = __builtin_fmaf((float)ov[r][c], (float)dv[r][c], acc);
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (ok[r] && sub == 0) {
      p.dsum[row[r]] = acc;
      p.lse2[row[r]] = (lv[r] == -INFINITY) ? -INFINITY : -lv[r] * kLog2e;
    }
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
    const int kr = (d == 128 ? 16 : 32) * kPreRep;   // rows per workgroup
    if (p.H <= 65535 && p.B <= 65535) {
      const dim3 grid((unsigned)((p.Nq + kr - 1) / kr), (unsigned)p.H, (unsigned)p.B);
      if (d == 128) hipLaunchKernelGGL((bwd_pre_kernel<16, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((bwd_pre_kernel<8, true>), grid, dim3(256), 0, s, p);
    } else {
      const dim3 grid((unsigned)((rows + kr - 1) / kr));
      if (d == 128) hipLaunchKernelGGL((bwd_pre_kernel<16, false>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((bwd_pre_kernel<8, false>), grid, dim3(256), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)(p.causal || p.local ? launch_bwd_masked(p, d, s) : launch_bwd_unmasked(p, d, s));
}

}  // namespace attn
