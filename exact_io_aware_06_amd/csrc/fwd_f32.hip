// Fused exact attention forward, float32 storage and float32 arithmetic
// throughout, for gfx950 (MI355X).
//
// The same streaming algorithm as the bf16 kernel (online softmax over
// key/value tiles held in LDS, "Understanding FlashAttention Pt 1: Personal
// Notes", sections 2.4 and 3.1), kept in full single precision: both
// contractions use v_mfma_f32_16x16x4_f32 and the probabilities stay fp32, so
// the only departures from exact arithmetic are fp32 roundings. This path is
// for small problems and accuracy checks, and laid out for latency.
//
//   * One workgroup = 16 query rows; its W = 8 wavefronts split the key
//     tiles among themselves (wave w takes tiles w, w+W, ...), each keeping its own running maximum, denominator and
//     output for the 16 rows, and the W partial results are merged through
//     LDS at the end (the merge of partial softmax results, "FlashAttention:
//     Mathematical Foundations...", section 7). At the small sizes this path
//     serves, one wave's chain of fp32 matrix instructions sets the time, so
//     spreading the keys of 16 rows over many waves shortens it.
//   * Scores transposed, S^T = K Q^T: in the 16x16 accumulator lane l holds
//     query l%16 and keys 4(l/16)..4(l/16)+3 of each 16-key block, so a row
//     reduction is in-lane plus two cross-lane steps (lanes l^16, l^32).
//   * O^T += V^T P^T: for the k = 4 contraction, lane group g supplies key
//     4g + i from accumulator register i; V is read as V[key][c] directly.
//   * K and Q go straight from memory into the MFMA operand registers as
//     16-byte vectors (the contraction over the head dimension is taken in
//     an order that makes each lane's four values adjacent); V is staged
//     per wave in its own part of LDS, so the waves never wait for one
//     another until the merge.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef ATTN_F32_WAVES_D64
#define ATTN_F32_WAVES_D64 8
#endif
#ifndef ATTN_F32_WAVES_D128
#define ATTN_F32_WAVES_D128 8
#endif
#ifndef ATTN_F32_KEYS_D64
#define ATTN_F32_KEYS_D64 32
#endif
#ifndef ATTN_F32_KEYS_D128
#define ATTN_F32_KEYS_D128 16
#endif
// Wavefronts per workgroup and keys per wave tile: 8 waves with 32-key
// tiles at d = 64 and 8 waves with 16-key tiles at d = 128 (a wave's V tile
// then takes 8.5 KB of LDS). On a single 256x256 head at d = 64, 8 waves
// ran 8.3 us against 8.8 us with 4 waves (64-key tiles) and 9.5 us with 16
// (16-key tiles): more waves shorten each wave's chain of matrix
// instructions but repeat the Q loads and lengthen the merge.
template <int D>
constexpr int f32_waves() { return D == 64 ? ATTN_F32_WAVES_D64 : ATTN_F32_WAVES_D128; }
template <int D>
constexpr int f32_keys() { return D == 64 ? ATTN_F32_KEYS_D64 : ATTN_F32_KEYS_D128; }
constexpr int kBr = 16;              // query rows per workgroup (all its waves)
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

// Orders one wave's LDS accesses across its lanes (a lane reads what
// another lane of the same wave wrote): the LDS queue of a wave is in order,
// so only the compiler has to be kept from moving accesses across this point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
__global__ __launch_bounds__(64 * f32_waves<D>()) void fwd_f32_kernel(FwdParams p, TileMap tm) {
  constexpr int kWaves = f32_waves<D>();
  constexpr int kBc = f32_keys<D>();      // keys per wave tile
  constexpr int kKb = kBc / 16;           // 16-key blocks of a tile
  constexpr int VP = D + 4;               // padded V row (floats): the rows
                                          // 4g + i of a PV step land on
                                          // distinct banks
  constexpr int NT = D / 16;              // 16-wide groups of the head dimension
  constexpr int NCB = D / 16;             // 16-wide output column blocks
  constexpr int kWaveFloats = kBc * VP;   // one wave's V tile
  static_assert(kWaveFloats % 4 == 0, "16-byte aligned V tiles");
  static_assert(kWaveFloats >= 16 * D + 32, "the merge reuses a wave's tile space");
  __shared__ __attribute__((aligned(16))) float lds[kWaves * kWaveFloats];

  int b, h, qt;
  if (!decode_tile(tm, p.B, p.H, b, h, qt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int hk = h / p.head_group;
  float* const vs = lds + wave * kWaveFloats;

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
  const int my_q = q0 + l16;
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

  // Q^T as the B operand. The contraction over the head dimension runs in
  // steps (t, i): at step (t, i) lane group g covers dimension 16t + 4g + i,
  // so each lane holds four consecutive dimensions of its row per t and
  // loads them as one 16-byte vector (K, the A operand, likewise).
  f32x4 qx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qx[t] = (my_q < Nq) ? *reinterpret_cast<const f32x4*>(qg + (int64_t)my_q * p.q_sn + 16 * t + 4 * g)
                        : f32x4{};

  f32x4 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) oacc[cb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;   // base-2 units
  const float c2 = p.scale_log2;
  const float* brow = nullptr;
  if (HAS_BIAS)
    brow = p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)min(my_q, Nq - 1) * p.bias_sn;

  for (int j = j0 + wave; j < nt; j += kWaves) {
    const int kv0 = j * kBc;
    if (p.local && kv0 + kBc <= q0 + off_l) continue;
    // K straight into registers in the A-operand layout (lane: key
    // kv0 + 16kb + l16, dimensions 16t + 4g .. +3); V through this wave's
    // LDS (chunk c: key c / (D/4), columns 4 (c % (D/4)) .. +3), since a PV
    // step wants it by column. Keys past Nk read as zeros. Every load of the
    // tile is issued before the first use, so the wave waits for memory
    // once per tile.
    constexpr int kChunks = kBc * D / 4 / 64;
    f32x4 kx[kKb][NT], vx[kChunks];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      const int key = kv0 + 16 * kb + l16;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        kx[kb][t] = (key < Nk) ? *reinterpret_cast<const f32x4*>(kgp + (int64_t)key * p.k_sn + 16 * t + 4 * g)
                               : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = lane + 64 * u;
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      vx[u] = (kv0 + key < Nk) ? *reinterpret_cast<const f32x4*>(vgp + (int64_t)(kv0 + key) * p.v_sn + col)
                               : f32x4{};
    }
    // the bias values of this lane's scores (keys kv0 + 16kb + 4g .. +3),
    // one 16-byte load when the row is aligned and all four keys exist
    f32x4 bv[kKb];
    if (HAS_BIAS) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        const int key = kv0 + 16 * kb + 4 * g;
        if (p.bias_vec && key + 3 < Nk) {
          bv[kb] = *reinterpret_cast<const f32x4*>(brow + key);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) bv[kb][i] = (key + i < Nk) ? brow[key + i] : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = lane + 64 * u;
      *reinterpret_cast<f32x4*>(&vs[(c / (D / 4)) * VP + (c % (D / 4)) * 4]) = vx[u];
    }
    wave_sync();

    // S^T blocks: register i of block kb holds key kv0 + 16kb + 4g + i
    f32x4 sacc[kKb];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) sacc[kb] = f32x4{};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kx[kb][t][i], qx[t][i], sacc[kb], 0, 0, 0);

#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kv0 + 16 * kb + 4 * g + i;
        float t;
        if (HAS_BIAS) {
          t = __builtin_fmaf(sacc[kb][i], c2, bv[kb][i] * kLog2e);
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
          const float a = vs[(16 * kb + 4 * g + i) * VP + 16 * cb + l16];
          oacc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sacc[kb][i], oacc[cb], 0, 0, 0);
        }
    wave_sync();  // the tile is read before the next one overwrites it
  }

  // ---- merge of the kWaves waves' partial results, through LDS: wave w
  // leaves O_w (unnormalised, 16 x D), m_w and l_w of each row in its own
  // tile space; then wave w finishes the column blocks cb = w, w + kWaves, ...:
  // with m = max_w m_w and s_w = 2^(m_w - m), O = sum_w s_w O_w / sum_w s_w l_w
  float l_w = l_run + __shfl_xor(l_run, 16);
  l_w = xor32_sum(l_w);
  float* const part = vs;                 // [16][D] then m[16], l[16]
  // register i of block cb holds column 16cb + 4g + i of row l16
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
    *reinterpret_cast<f32x4*>(&part[l16 * D + 16 * cb + 4 * g]) = oacc[cb];
  if (g == 0) {
    part[16 * D + l16] = m_run;
    part[16 * D + 16 + l16] = l_w;
  }
  __syncthreads();
  float mw[kWaves], sw[kWaves];
  float m_all = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = lds[w * kWaveFloats + 16 * D + l16];
    m_all = fmaxf(m_all, mw[w]);
  }
  float l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    sw[w] = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - m_all);
    l_tot += sw[w] * lds[w * kWaveFloats + 16 * D + 16 + l16];
  }
  if (my_q < Nq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = static_cast<float*>(p.o) + (varlen ? q_lo * p.o_sn : b * p.o_sb) + h * p.o_sh +
                  (int64_t)my_q * p.o_sn;
    for (int cb = wave; cb < NCB; cb += kWaves) {
      f32x4 acc{};
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        acc += sw[w] * *reinterpret_cast<const f32x4*>(&lds[w * kWaveFloats + l16 * D + 16 * cb + 4 * g]);
      *reinterpret_cast<f32x4*>(orow + 16 * cb + 4 * g) = acc * inv;
    }
    if (wave == 0 && g == 0) {
      float* lrow = p.lse + (varlen ? q_lo : b * p.l_sb) + h * p.l_sh;
      lrow[my_q] = (l_tot > 0.f) ? (m_all + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool HAS_BIAS>
hipError_t launch_one(const FwdParams& p, const TileMap& tm, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, HAS_BIAS>), dim3(8 * tm.per_xcd),
                     dim3(64 * f32_waves<D>()), 0, stream, p, tm);
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
