// Fused exact attention forward, bfloat16 storage, for gfx950 (MI355X).
//
// What is computed: O = softmax_row(scale * Q K^T + Bias) V and the per-row
// natural log-sum-exp, with the score tile consumed on chip by the online
// softmax recurrence ("Understanding FlashAttention Pt 1: Personal Notes",
// sections 2.3-2.4 and 3.1). The loop order is query tile outermost with the
// unnormalised output kept in registers and divided once at the end
// ("FlashAttention: Mathematical Foundations...", section 5, loop inversion;
// "FlashAttention, Explained", section 20). Exponentials are base 2 with the
// softmax scale folded into one fused multiply-add per score
// ("flash-attention", stanleyjacob.dev, Part VI).
//
// Work decomposition on CDNA4
//   * One workgroup = 4 wavefronts = 128 query rows of one (batch, head);
//     each wavefront owns 32 rows, so no cross-wave reduction of O is needed.
//   * Key/value tiles of 64 keys are staged global -> registers -> LDS, double
//     buffered: the global loads of tile j+1 are issued before tile j is
//     computed and land in the other LDS buffer afterwards; one barrier per
//     tile.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys from LDS, B = 32 queries held in
//     VGPRs for the whole loop). In the 32x32 accumulator layout lane l holds
//     query l%32 and 16 of the 32 keys; the other 16 sit in lane l^32. A row
//     maximum is therefore 31 in-lane max operations and ONE cross-lane step
//     (v_permlane32_swap); the row sum needs no cross-lane step until the end.
//   * The rows of the K operand are fed in a fixed permutation (bits 2 and 3
//     of the row index swapped) so that the accumulator registers 8t..8t+7 of
//     every lane hold 8 consecutive keys. They are converted to bf16 in place
//     and used directly as the B operand of O^T += V^T P^T, with no shuffle.
//   * V is written to LDS key-interleaved: the 16-byte unit (g, c) holds
//     V[8g..8g+7][c], which is exactly one lane's A operand of the PV MFMA.
//     The interleave is done in registers by the loader threads.
//   * K rows are stored in LDS in the permuted order with a 16-byte row pad so
//     the 32 rows read by one MFMA operand fall in distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_params.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per tile
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

template <int D>
struct Geo {
  static constexpr int kRowBytes = D * 2 + 16;        // padded K row in LDS
  static constexpr int kKBytes = kBc * kRowBytes;
  static constexpr int kVBytes = kBc * D * 2;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kSmem = 2 * kStage;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kKLoads = kBc * kChunks / kThreads;
  static constexpr int kVCols = D / 32;               // V columns per loader thread
  static constexpr int kNkk = D / 16;                 // k-steps of QK^T
  static constexpr int kNcb = D / 32;                 // 32-wide output column blocks
};

// Row permutation of the K operand: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float lane_pair_max(float x) {
  // lanes l and l^32 end up holding max(x_l, x_{l^32})
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float x) {
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

template <int D>
struct VLoad;
template <>
struct VLoad<128> { typedef u32x2 type; };   // 4 columns = 8 bytes
template <>
struct VLoad<64> { typedef uint32_t type; }; // 2 columns = 4 bytes

__device__ __forceinline__ uint32_t word_of(const u32x2& v, int i) { return v[i]; }
__device__ __forceinline__ uint32_t word_of(const uint32_t& v, int) { return v; }

template <int D, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdParams p, TileMap tm) {
  using G = Geo<D>;
  using VRow = typename VLoad<D>::type;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  int b, h, qt;
  if (!decode_tile(tm, p.B, p.H, b, h, qt)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int hk = h / p.head_group;

  const __bf16* qg = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kgp = static_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const __bf16* vgp = static_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh;

  const int Nq = p.Nq;
  const int Nk = p.Nk;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const int off = Nk - Nq;  // causal alignment: key j hidden when j > i + off

  int kend = Nk;
  if (p.kv_len != nullptr) kend = min(max(p.kv_len[b], 0), Nk);
  int wg_keys = kend;
  if (CAUSAL) wg_keys = min(kend, min(q0 + kBr, Nq) + off);
  wg_keys = max(wg_keys, 0);
  const int nt = (wg_keys + kBc - 1) / kBc;
  int wave_keys = 0;
  if (qw0 < Nq) {
    wave_keys = kend;
    if (CAUSAL) wave_keys = min(kend, min(qw0 + 32, Nq) + off);
    wave_keys = max(wave_keys, 0);
  }

  // ---- Q as the B operand, resident for the whole loop: lane holds query
  // my_q, elements [16kk + 8hi, 16kk + 8hi + 8).
  bf16x8 qf[G::kNkk];
  if (my_q < Nq) {
    const __bf16* qrow = qg + (int64_t)my_q * p.q_sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < G::kNkk; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < G::kNkk; ++kk)
      qf[kk] = bf16x8{};
  }

  // ---- loader roles
  // K: chunk c = tid + kThreads*i -> key c / kChunks, 16-byte column chunk c % kChunks
  // V: key group g = tid / 32 (8 keys), columns [vc0, vc0 + kVCols)
  const int vg = tid >> 5;
  const int vc0 = (tid & 31) * G::kVCols;
  u32x4 kreg[G::kKLoads];
  VRow vreg[8];

  auto load_tile = [&](int j) {
    const int kv0 = j * kBc;
    const bool full = kv0 + kBc <= Nk;
#pragma unroll
    for (int i = 0; i < G::kKLoads; ++i) {
      const int c = tid + kThreads * i;
      const int key = kv0 + c / G::kChunks;
      const int ch = c % G::kChunks;
      if (full || key < Nk)
        kreg[i] = *reinterpret_cast<const u32x4*>(kgp + (int64_t)key * p.k_sn + ch * 8);
      else
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = kv0 + vg * 8 + r;
      if (full || key < Nk)
        vreg[r] = *reinterpret_cast<const VRow*>(vgp + (int64_t)key * p.v_sn + vc0);
      else
        vreg[r] = VRow{};
    }
  };

  auto store_tile = [&](int stage) {
    uint8_t* ks = smem + stage * G::kStage;
    uint8_t* vs = ks + G::kKBytes;
#pragma unroll
    for (int i = 0; i < G::kKLoads; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / G::kChunks;
      const int ch = c % G::kChunks;
      const int row = (key & ~31) | perm_row(key & 31);
      *reinterpret_cast<u32x4*>(ks + row * G::kRowBytes + ch * 16) = kreg[i];
    }
    // key-interleave V: unit (vg, c) = V[8vg .. 8vg+7][c]
#pragma unroll
    for (int cc = 0; cc < G::kVCols; ++cc) {
      u32x4 u;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint32_t lo = word_of(vreg[2 * pp], cc >> 1);
        const uint32_t up = word_of(vreg[2 * pp + 1], cc >> 1);
        u[pp] = (cc & 1) ? ((lo >> 16) | (up & 0xffff0000u))
                         : ((lo & 0xffffu) | (up << 16));
      }
      *reinterpret_cast<u32x4*>(vs + (vg * D + vc0 + cc) * 16) = u;
    }
  };

  // ---- running state of this lane's query row
  f32x16 oacc[G::kNcb];
#pragma unroll
  for (int cb = 0; cb < G::kNcb; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;  // running maximum, base-2 units
  float l_run = 0.f;        // this lane's share of the running denominator
  const float c2 = p.scale_log2;

  const float* brow = nullptr;
  if (HAS_BIAS) {
    const int qrow = min(my_q, Nq - 1);
    brow = p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)qrow * p.bias_sn + 8 * hi;
  }

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }

  for (int j = 0; j < nt; ++j) {
    const int stage = j & 1;
    if (j + 1 < nt) load_tile(j + 1);

    const int kv0 = j * kBc;
    if (kv0 < wave_keys) {
      const uint8_t* ks = smem + stage * G::kStage;
      const uint8_t* vs = ks + G::kKBytes;

      f32x16 bia[2];
      if (HAS_BIAS) {
        // lane's keys in block bb: kv0 + 32bb + 16s + 8hi + [0, 8), s = 0, 1
        const bool fullb = p.bias_vec && kv0 + kBc <= Nk;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const float* src = brow + kv0 + 32 * bb + 16 * s;
            if (fullb) {
              const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
              const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                bia[bb][8 * s + e] = x0[e];
                bia[bb][8 * s + 4 + e] = x1[e];
              }
            } else {
              const int k0 = kv0 + 32 * bb + 16 * s + 8 * hi;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                bia[bb][8 * s + e] = (k0 + e < Nk) ? src[e] : 0.f;
            }
          }
      }

      // ---- S^T = K Q^T for two 32-key blocks
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      const uint8_t* kbase = ks + l32 * G::kRowBytes + hi * 16;
#pragma unroll
      for (int kk = 0; kk < G::kNkk; ++kk)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kbase + bb * 32 * G::kRowBytes + kk * 32);
          sacc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[bb], 0, 0, 0);
        }

      // register r of block bb holds key kv0 + 32bb + 16(r/8) + 8hi + (r%8)
      if (HAS_BIAS) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[bb][r] = __builtin_fmaf(sacc[bb][r], c2, bia[bb][r] * kLog2e);
      }
      const bool need_mask = (kv0 + kBc > kend) || (CAUSAL && kv0 + kBc - 1 > qw0 + off);
      if (need_mask) {
        const int lim_c = my_q + off;  // last key this query may see (causal)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
            const bool hide = (key >= kend) || (CAUSAL && key > lim_c);
            if (hide) sacc[bb][r] = -INFINITY;
          }
      }

      // ---- online softmax update (base 2)
      float mx = sacc[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
      mx = lane_pair_max(mx);
      const float m_new = HAS_BIAS ? fmaxf(m_run, mx) : fmaxf(m_run, mx * c2);
      // a row with nothing visible yet keeps 0 as its reference (no -inf - -inf)
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

      float rs = 0.f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = HAS_BIAS ? (sacc[bb][r] - m_use)
                                   : __builtin_fmaf(sacc[bb][r], c2, -m_use);
          const float e = __builtin_amdgcn_exp2f(t);
          sacc[bb][r] = e;
          rs += e;
        }
      l_run = __builtin_fmaf(l_run, alpha, rs);
      m_run = m_new;
      // rescale the accumulator only if some row of this wave moved its maximum
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      }

      // ---- P^T operands: registers 8t..8t+7 of block bb = keys 32bb+16t+8hi+[0,8)
      bf16x8 pb[2][2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[bb][t][e] = (__bf16)sacc[bb][8 * t + e];

      // ---- O^T += V^T P^T
      const uint8_t* vbase = vs + (hi * D + l32) * 16;
#pragma unroll
      for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                vbase + ((4 * bb + 2 * t) * D + 32 * cb) * 16);
            oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[bb][t], oacc[cb], 0, 0, 0);
          }
    }

    if (j + 1 < nt) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one division per row, O and LSE written once
  const float l_tot = lane_pair_sum(l_run);
  if (my_q < Nq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    __bf16* orow = static_cast<__bf16*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)my_q * p.o_sn;
    // register r of block cb holds column 32cb + 8(r/4) + 4hi + (r%4)
#pragma unroll
    for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[cb][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * g + 4 * hi) = w;
      }
    if (hi == 0) {
      float* lrow = p.lse + b * p.l_sb + h * p.l_sh;
      lrow[my_q] = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool HAS_BIAS>
hipError_t launch_one(const FwdParams& p, const TileMap& tm, hipStream_t stream) {
  using G = Geo<D>;
  static bool attr_set = false;  // benign race: every caller sets the same value
  auto kern = fwd_bf16_kernel<D, CAUSAL, HAS_BIAS>;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, G::kSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = 8 * tm.per_xcd;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), G::kSmem, stream, p, tm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, const TileMap& tm, hipStream_t s) {
  const bool bias = p.bias != nullptr;
  if (p.causal) return bias ? launch_one<D, true, true>(p, tm, s) : launch_one<D, true, false>(p, tm, s);
  return bias ? launch_one<D, false, true>(p, tm, s) : launch_one<D, false, false>(p, tm, s);
}

}  // namespace

int launch_fwd_bf16(const FwdParams& p, int d, void* stream) {
  TileMap tm;
  tm.n_qtiles = (p.Nq + kBr - 1) / kBr;
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
