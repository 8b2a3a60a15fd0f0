// Fused exact attention forward, float32 storage and float32 arithmetic
// throughout, for gfx950 (MI355X).
//
// The same streaming algorithm as the bf16 kernel (online softmax over
// key/value tiles held in LDS, "Understanding FlashAttention Pt 1: Personal
// Notes", sections 2.4 and 3.1), kept in full single precision: both
// contractions use v_mfma_f32_16x16x4_f32 and the probabilities stay fp32, so
// the only departures from exact arithmetic are fp32 roundings. This path is
// for small problems and accuracy checks; it is latency-bound, not tuned.
//
//   * One workgroup = 4 wavefronts x 16 query rows; tiles of 64 keys.
//   * Scores transposed, S^T = K Q^T: in the 16x16 accumulator lane l holds
//     query l%16 and keys 4(l/16)..4(l/16)+3 of each 16-key block, so a row
//     reduction is in-lane plus two cross-lane steps (lanes l^16, l^32).
//   * O^T += V^T P^T: for the k = 4 contraction, lane group g supplies key
//     4g + i from accumulator register i; V is read as V[key][c] directly.
//   * Single-buffered LDS; the next tile is loaded into registers while the
//     current one is computed (load latency, not arithmetic, bounds the
//     small problems this path serves), then stored to LDS between two
//     barriers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 16 * kWaves;
constexpr int kBc = 64;
constexpr int kKb = kBc / 16;   // 16-key blocks of a tile
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool decode_tile(const TileMap& tm, int B, int H,
                                            int& b, int& h, int& qt) {
  const int w = blockIdx.x;
  const int logical = (w & 7) * tm.per_xcd + (w >> 3);
  if (logical >= tm.total) return false;
  int rest;
  int qi;
  if (tm.batch_inner) {
    b = logical % B;
    rest = logical / B;
    qi = rest % tm.n_qtiles;
    h = rest / tm.n_qtiles;
  } else {
    qi = logical % tm.n_qtiles;
    rest = logical / tm.n_qtiles;
    h = rest % H;
    b = rest / H;
  }
  qt = tm.reverse_q ? (tm.n_qtiles - 1 - qi) : qi;
  return true;
}

template <int D, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdParams p, TileMap tm) {
  constexpr int KP = D + 1;             // padded K row (floats)
  constexpr int NS = D / 4;             // k-steps of QK^T
  constexpr int NCB = D / 16;           // 16-wide output column blocks
  __shared__ float ks[kBc * KP];
  __shared__ __attribute__((aligned(16))) float vs[kBc * D];

  int b, h, qt;
  if (!decode_tile(tm, p.B, p.H, b, h, qt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int hk = h / p.head_group;

  // packed variable-length sequences: b is a sequence with rows [q_lo,
  // q_lo + Nq) and keys [k_lo, k_lo + Nk) of the packed tensors (offsets
  // clamped into the tensors)
  int Nq = p.Nq, Nk = p.Nk;
  int64_t q_lo = 0, k_lo = 0;
  const bool varlen = p.cu_q != nullptr;
  if (varlen) {
    const int a0 = min(max(p.cu_q[b], 0), p.Nq), a1 = min(max(p.cu_q[b + 1], a0), p.Nq);
    const int c0 = min(max(p.cu_k[b], 0), p.Nk), c1 = min(max(p.cu_k[b + 1], c0), p.Nk);
    q_lo = a0;
    Nq = a1 - a0;
    k_lo = c0;
    Nk = c1 - c0;
    if (qt * kBr >= Nq) return;
  }
  const float* qg = static_cast<const float*>(p.q) + (varlen ? q_lo * p.q_sn : b * p.q_sb) + h * p.q_sh;
  const float* kgp = static_cast<const float*>(p.k) + (varlen ? k_lo * p.k_sn : b * p.k_sb) + hk * p.k_sh;
  const float* vgp = static_cast<const float*>(p.v) + (varlen ? k_lo * p.v_sn : b * p.v_sb) + hk * p.v_sh;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 16;
  const int my_q = qw0 + l16;
  // causal alignment: key j hidden from query i when j > i + off; with a
  // window (p.local, on the causal instantiations) also when j < i + off_l
  const int off = Nk - Nq + (p.local ? p.win_right : 0);
  const int off_l = Nk - Nq - p.win_left;
  // first tile any row of this workgroup may see
  const int j0 = p.local ? max(q0 + off_l, 0) / kBc : 0;

  int kend = Nk;
  if (p.kv_len != nullptr) kend = min(max(p.kv_len[b], 0), Nk);
  int wg_keys = kend;
  if (CAUSAL) wg_keys = min(kend, min(q0 + kBr, Nq) + off);
  wg_keys = max(wg_keys, 0);
  const int nt = (wg_keys + kBc - 1) / kBc;
  int wave_keys = 0;
  if (qw0 < Nq) {
    wave_keys = kend;
    if (CAUSAL) wave_keys = min(kend, min(qw0 + 16, Nq) + off);
    wave_keys = max(wave_keys, 0);
  }

  // Q^T as the B operand: lane holds Q[my_q][4s + g] for every k-step s
  float qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = (my_q < Nq) ? qg[(int64_t)my_q * p.q_sn + 4 * s + g] : 0.f;

  f32x4 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;
  const float* brow = nullptr;
  if (HAS_BIAS)
    brow = p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)min(my_q, Nq - 1) * p.bias_sn;

  // chunk c of a tile (c = tid + kThreads * n): key c / (D/4), columns
  // 4 (c % (D/4)) .. +3; keys past Nk read as zeros
  constexpr int kChunks = kBc * D / 4 / kThreads;
  f32x4 kx[kChunks], vx[kChunks];
  auto fetch = [&](int j) {
    const int kv0 = j * kBc;
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
      const int c = tid + kThreads * n;
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      kx[n] = f32x4{};
      vx[n] = f32x4{};
      if (kv0 + key < Nk) {
        kx[n] = *reinterpret_cast<const f32x4*>(kgp + (int64_t)(kv0 + key) * p.k_sn + col);
        vx[n] = *reinterpret_cast<const f32x4*>(vgp + (int64_t)(kv0 + key) * p.v_sn + col);
      }
    }
  };
  if (j0 < nt) fetch(j0);
  for (int j = j0; j < nt; ++j) {
    const int kv0 = j * kBc;
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
      const int c = tid + kThreads * n;
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[key * KP + col + e] = kx[n][e];
      *reinterpret_cast<f32x4*>(&vs[key * D + col]) = vx[n];
    }
    if (j + 1 < nt) fetch(j + 1);
    __syncthreads();
    if (kv0 >= wave_keys || (p.local && kv0 + kBc <= qw0 + off_l)) continue;

    // S^T blocks: register i of block kb holds key kv0 + 16kb + 4g + i
    f32x4 sacc[kKb];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) sacc[kb] = f32x4{};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        const float a = ks[(16 * kb + l16) * KP + 4 * s + g];
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[s], sacc[kb], 0, 0, 0);
      }

#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kv0 + 16 * kb + 4 * g + i;
        float t;
        if (HAS_BIAS) {
          const float bv = (key < Nk) ? brow[key] : 0.f;
          t = __builtin_fmaf(sacc[kb][i], c2, bv * kLog2e);
        } else {
          t = sacc[kb][i] * c2;
        }
        const bool hide = (key >= kend) || (CAUSAL && key > my_q + off) ||
                          (p.local && key < my_q + off_l);
        sacc[kb][i] = hide ? -INFINITY : t;
      }

    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(sacc[kb][i] - m_use);
        sacc[kb][i] = e;
        rs += e;
      }
    l_run = __builtin_fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) oacc[cb] *= alpha;

    // O^T += V^T P^T, one key per lane group per MFMA
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = vs[(16 * kb + 4 * g + i) * D + 16 * cb + l16];
          oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sacc[kb][i], oacc[cb], 0, 0, 0);
        }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot = xor32_sum(l_tot);
  if (my_q < Nq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = static_cast<float*>(p.o) + (varlen ? q_lo * p.o_sn : b * p.o_sb) + h * p.o_sh +
                  (int64_t)my_q * p.o_sn;
    // register i of block cb holds column 16cb + 4g + i
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      *reinterpret_cast<f32x4*>(orow + 16 * cb + 4 * g) = oacc[cb] * inv;
    if (g == 0) {
      float* lrow = p.lse + (varlen ? q_lo : b * p.l_sb) + h * p.l_sh;
      lrow[my_q] = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool HAS_BIAS>
hipError_t launch_one(const FwdParams& p, const TileMap& tm, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, HAS_BIAS>), dim3(8 * tm.per_xcd),
                     dim3(kThreads), 0, stream, p, tm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, const TileMap& tm, hipStream_t s) {
  const bool bias = p.bias != nullptr;
  if (p.causal) return bias ? launch_one<D, true, true>(p, tm, s) : launch_one<D, true, false>(p, tm, s);
  return bias ? launch_one<D, false, true>(p, tm, s) : launch_one<D, false, false>(p, tm, s);
}

}  // namespace

int launch_fwd_f32(const FwdParams& p, int d, void* stream) {
  TileMap tm{};
  tm.n_qtiles = ((p.cu_q != nullptr ? p.max_q : p.Nq) + kBr - 1) / kBr;
  const int64_t total = (int64_t)p.B * p.H * tm.n_qtiles;
  tm.total = (int)total;
  tm.per_xcd = (int)((total + 7) / 8);
  tm.batch_inner = (p.bias != nullptr && p.bias_sb == 0 && p.B > 1) ? 1 : 0;
  tm.reverse_q = p.causal ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 128) return (int)launch_d<128>(p, tm, s);
  if (d == 64) return (int)launch_d<64>(p, tm, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace attn
