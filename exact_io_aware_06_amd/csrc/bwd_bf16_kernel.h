// Attention backward with recomputation, bfloat16 storage, gfx950 (MI355X):
// kernel templates and the per-variant launcher. Instantiated in
// bwd_bf16.hip (no mask edge: the preprocess, the dispatch and the
// unmasked variants) and bwd_bf16_masked.hip (causal and window variants).
//
// What is computed: for an upstream gradient dO of O = softmax_row(S) V with
// S = scale * Q K^T + Bias (masks as -inf),
//     D_i = rowsum(dO_i o O_i),      P_ij = exp(S_ij - LSE_i),
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//     dQ = scale * dS K,             dK = scale * dS^T Q.
// P is never stored: each tile of it is rebuilt from Q, K and the forward's
// log-sum-exp, which makes every tile self-contained ("Understanding
// FlashAttention Pt 1", section 3.6; "FlashAttention, Explained", sections
// 16-17, including the identity rowsum(dP o P) = rowsum(dO o O) that D uses;
// "FlashAttention: Mathematical Foundations...", section 4; "flash-attention"
// (stanleyjacob.dev), Part VII, the preprocess pass and P = exp(S - LSE)).
//
// Work decomposition on CDNA4 (three launches):
//   * preprocess: d/8 lanes per query row (16-byte loads of O and dO)
//     write D and the negated log-sum-exp in base 2 (-inf for a row that
//     saw no key, so every probability it recomputes is exactly 0; negated
//     so that the exponent log2(e) S - LSE2 is one fused multiply-add);
//   * dK/dV: one workgroup = 4 wavefronts = 128 keys of one (batch, K/V
//     head); each wavefront owns 32 keys and keeps their K and V rows and
//     dK^T, dV^T in registers while Q, dO tiles of 64 query rows stream
//     through LDS (all query heads of the group, so grouped heads sum in
//     registers; the tiles use a bank-rotated variant of the forward's K
//     layout, below). S = Q K^T and dP = dO V^T are computed with the key in the
//     lane (the query rows are fed in the bits-2/3 permuted order, so the
//     accumulator registers 8t..8t+7 hold 8 consecutive queries): P and dS,
//     converted to bf16 in place, are directly the B operands of
//     dV^T += dO^T P and dK^T += Q^T dS, whose A operands are read from the
//     Q / dO tiles with LDS transpose reads.
//   * dQ: one workgroup = 4 wavefronts = 128 query rows; the forward's
//     layout (S^T = K Q^T and dP^T = V dO^T with the query in the lane, Q and
//     dO rows resident as B operands), dS^T feeding dQ^T += K^T dS^T with K^T
//     read from the K tile by LDS transpose reads.
// dQ is produced by its own query-parallel pass instead of atomic additions
// from the key-parallel one: that recomputes S and dP (7 tile products
// instead of 5), but the result is deterministic and no fp32 atomics are
// issued per element of dQ per key tile.

#pragma once

#include "fwd_bf16_kernel.h"

namespace attn {
namespace {

constexpr int kBt = 64;  // rows of one streamed tile (queries in dK/dV, keys in dQ)

// LDS tile layout of the backward ("rotated"): blocks of 16 rows; in a
// block, 16-byte chunk c of row r sits at slot 16c + ((r + 4c) mod 16), and
// LDS row R holds tile row perm_row(R) (bits 2 and 3 swapped) as in the
// forward's K tiles. Every tile is read two ways: as rows (A operands of S
// and dP: 16 lanes read 16 rows of one chunk) and transposed (A operands of
// the dV, dK, dQ products: ds_read_b64_tr_b16 over 4 rows x 4 chunks x 2
// column groups per 32 lanes). Without the rotation the chunks of a
// transposed read fall on the same 16 banks (a 4-way conflict); rotating
// each chunk's rows by 4c spreads both kinds of read over all 64 banks.
//
// Source row of the 16 bytes that `lane` of wave `wave` copies in DMA
// instruction i (instruction n writes LDS bytes [1024 n, 1024 n + 1024),
// lane l at 16 l); the byte column is k_dma_col's.
template <int D, int W>
__device__ __forceinline__ int rot_dma_row(int wave, int lane, int i) {
  const int a = 1024 * (wave + W * i) + 16 * lane;
  constexpr int blk = 16 * (D / 8) * 16;
  const int slot = (a % blk) / 16;
  const int c = slot / 16;
  return perm_row(16 * (a / blk) + ((slot % 16 - 4 * c) & 15));
}

// DMA instruction i + 1 of a wave copies the rows of instruction i moved on
// by a fixed step, at the same byte column: its LDS bytes lie W KB further,
// a whole number of 16-row blocks. So one row and one column per lane
// describe all of a wave's copies of a tile.
template <int D, int W>
constexpr int dma_row_step() {
  static_assert((W * 1024) % (32 * D) == 0, "a wave's copies must advance by whole 16-row blocks");
  return 16 * (W * 1024) / (32 * D);
}


// Row read (A operand) of chunk pair kk: lane-constant offset for even and
// odd kk (the rotation of chunk 2kk + hi is 8kk + 4hi mod 16); the caller
// adds 2 mbq * block + 512 kk.
__device__ __forceinline__ int row_lane_offset(int lane, int G_block, int odd) {
  const int l32 = lane & 31, hi = lane >> 5;
  return (l32 >> 4) * G_block + 256 * hi + 16 * (((l32 & 15) + 4 * hi + 8 * odd) & 15);
}

// Transposed read: within its 16-lane group, lane 4e + j addresses tile row
// e + 4 hi (+ 8 for the second read of a pair), columns 4j..4j+3 of the
// group's 16 columns; lane-constant offset of each read of the pair. The
// caller adds block and 1024 * (32-column block) offsets.
__device__ __forceinline__ int tr_lane_offset(int lane, int half) {
  const int L = lane & 15, e = L >> 2, j = L & 3, g = (lane >> 4) & 1, hi = lane >> 5;
  return 256 * (2 * g + (j >> 1)) + 16 * ((e + 4 * hi + 8 * g + 4 * (j >> 1) + 8 * half) & 15) +
         8 * (j & 1);
}


// ------------------------------------------------------------- dK and dV
// Two workgroups per CU (two wavefronts per SIMD), so one wavefront's
// exponentials overlap the other's matrix products; at d = 128 that keeps
// the kernel within 256 registers (the variants with a bias or a window
// spill a few dwords) and was measured 1.31x faster than one wavefront per
// SIMD with no register limit.
template <int D, int W, bool CAUSAL, bool HAS_BIAS, bool LOCAL>
__global__ __launch_bounds__(64 * W, 2) void bwd_dkdv_kernel(BwdParams p, TileMap tm) {
  using G = Geo<D, W>;
  constexpr int kNkk = D / 16;   // d-steps of S and dP
  constexpr int kNcb = D / 32;   // d blocks of dK^T, dV^T
  constexpr int kStage = 2 * G::kKBytes + 2 * kBt * 4;  // Q tile, dO tile, lse2[64], D[64]
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // key tile fastest (neighbouring key tiles read the same Q / dO), then
  // K/V head, batch; causal: heads dealt in small groups with the key tile
  // slow inside a group; consecutive logical tiles share an XCD
  const int w = blockIdx.x;
  const int logical = (w & 7) * tm.per_xcd + (w >> 3);
  if (logical >= tm.total) return;
  int kt, hb;  // causal: key tile 0 sees the most queries (longest first)
  split_logical(logical, tm.n_qtiles, p.B * p.Hk, tm.group, kt, hb);
  const int hk = hb % p.Hk;
  const int b = hb / p.Hk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;
  const int k0 = kt * 32 * W;
  const int my_k = k0 + wave * 32 + l32;  // this lane's key
  int kend = Nk;
  if (p.kv_len != nullptr) kend = min(max(p.kv_len[b], 0), Nk);
  const int off = Nk - Nq + (LOCAL ? p.win_right : 0);  // key j hidden from query i if j > i + off
  const int off_l = Nk - Nq - p.win_left;               // (window) ... or if j < i + off_l
  const float c2 = p.scale_log2;

  // K and V rows of this lane's key, resident: B operands of S and dP
  bf16x8 kf[kNkk], vf[kNkk];
  {
    const int kr = min(my_k, Nk - 1);
    const __bf16* krow = static_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)kr * p.k_sn + 8 * hi;
    const __bf16* vrow = static_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)kr * p.v_sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kNkk; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
      vf[kk] = *reinterpret_cast<const bf16x8*>(vrow + 16 * kk);
    }
  }

  // Query rows that can see any key of this workgroup, whole 64-row tiles
  int q_lo = 0, q_hi = Nq;
  if (CAUSAL) q_lo = max(0, k0 - off);                       // i >= j - off
  if (LOCAL) q_hi = min(Nq, k0 + 32 * W - off_l);            // i <= j - off_l
  if (k0 >= kend) q_hi = 0;                                  // no visible key at all
  q_lo = q_lo / kBt * kBt;
  const int nqb = q_hi > q_lo ? (q_hi - q_lo + kBt - 1) / kBt : 0;
  const int ns = nqb * p.head_group;  // stages: (query head of the group, query tile)

  // LDS DMA sources: instruction i of this wave copies 16 bytes of tile row
  // rrow0 + kRowStep * i (the rotated layout's permuted row), byte column
  // rcol. Two registers instead of one pair per instruction: kept across the
  // stage loop, per-instruction values were spilled and reloaded each stage.
  constexpr int kRowStep = dma_row_step<D, W>();
  const int rrow0 = rot_dma_row<D, W>(wave, lane, 0);
  const int rcol = k_dma_col<D, W>(wave, lane, 0);
  const int64_t qsn = p.q_sn * 2, dsn = p.do_sn * 2;  // row strides in bytes
  auto stage_head = [&](int s) { return hk * p.head_group + s / nqb; };
  auto stage_q0 = [&](int s) { return q_lo + (s % nqb) * kBt; };
  // copy the Q and dO tiles of stage s into buffer `buf` (rows past Nq read
  // row Nq - 1: finite data whose probabilities are 0, their -LSE2 being -inf)
  auto issue = [&](int s, int buf) {
    const int h = stage_head(s), q0 = stage_q0(s);
    const int lim = Nq - 1 - q0;
    const uint8_t* qt = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh) + q0 * qsn;
    const uint8_t* dt = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.do_) + b * p.do_sb + h * p.do_sh) + q0 * dsn;
    uint8_t* st = smem + buf * kStage;
    const int r0 = fresh(rrow0);
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i) {
      const int r = min(r0 + kRowStep * i, lim);
      dma16(qt, (uint32_t)(r * (int)qsn + rcol), st + 1024 * (wave + W * i));
      dma16(dt, (uint32_t)(r * (int)dsn + rcol), st + G::kKBytes + 1024 * (wave + W * i));
    }
  };
  // negated base-2 LSE (wave 0) and D (wave 1) of stage s: one value per lane
  auto load_stats = [&](int s) {
    const int h = stage_head(s), qi = stage_q0(s) + fresh(lane);
    const int64_t row = ((int64_t)b * p.H + h) * Nq + min(qi, Nq - 1);
    float x = 0.f;
    if (wave == 0) x = (qi < Nq) ? p.lse2[row] : -INFINITY;
    else if (wave == 1) x = (qi < Nq) ? p.dsum[row] : 0.f;
    return x;
  };
  auto store_stats = [&](int buf, float x) {
    float* st = reinterpret_cast<float*>(smem + buf * kStage + 2 * G::kKBytes);
    const int ln = fresh(lane);
    if (wave == 0) st[ln] = x;
    else if (wave == 1) st[kBt + ln] = x;
  };
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 dk_acc[kNcb], dv_acc[kNcb];
#pragma unroll
  for (int mb = 0; mb < kNcb; ++mb) {
    dk_acc[mb] = f32x16{};
    dv_acc[mb] = f32x16{};
  }
  // LDS read offsets: rows (A operands of S and dP) and transposed reads
  const int rl0 = row_lane_offset(lane, G::kKBlock, 0), rl1 = row_lane_offset(lane, G::kKBlock, 1);
  const int tl0 = tr_lane_offset(lane, 0), tl1 = tr_lane_offset(lane, 1);

  if (ns > 0) {
    issue(0, 0);
    store_stats(0, load_stats(0));
    wait_tiles();
    __syncthreads();
  }
  for (int s = 0; s < ns; ++s) {
    const int buf = s & 1;
    float nxt = 0.f;
    if (s + 1 < ns) {
      issue(s + 1, buf ^ 1);
      nxt = load_stats(s + 1);
    }
    const int h = stage_head(s), q0 = stage_q0(s);
    const uint8_t* Qt = smem + buf * kStage;
    const uint8_t* dOt = Qt + G::kKBytes;
    const float* lt = reinterpret_cast<const float*>(Qt + 2 * G::kKBytes) + fresh(8 * hi);
    const float* dtv = lt + kBt;
    const float* brow = nullptr;
    if (HAS_BIAS) brow = p.bias + b * p.bias_sb + h * p.bias_sh + min(my_k, Nk - 1);
#pragma unroll
    for (int mbq = 0; mbq < 2; ++mbq) {
      // S = Q K^T and dP = dO V^T for 32 queries (rows) x this lane's key
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < kNkk; ++kk) {
        const int ro = (kk & 1 ? rl1 : rl0) + mbq * 2 * G::kKBlock + kk * 512;
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qt + ro);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dOt + ro);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vf[kk], pacc, 0, 0, 0);
      }
      // register r holds query q0 + 32 mbq + 16 (r / 8) + 8 hi + (r % 8).
      // Keys past the key length are not masked: a key feeds only its own
      // column of dK^T and dV^T, which the epilogue writes as zeros.
      const int qb = q0 + 32 * mbq + 8 * hi;
      const bool need_mask = (CAUSAL && k0 + 32 * W - 1 > q0 + 32 * mbq + off) ||
                             (LOCAL && k0 < q0 + 32 * mbq + 31 + off_l);
      // hidden scores become -inf in place (scale > 0, so the exponent
      // below stays -inf and P = 0); only tiles that cross the mask's edge
      // take this branch
      if ((CAUSAL || LOCAL) && need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qb + 16 * (r >> 3) + (r & 7);
          if ((CAUSAL && my_k > qi + off) || (LOCAL && my_k < qi + off_l)) sacc[r] = -INFINITY;
        }
      }
      u32x4 pb[2], db[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lt + 32 * mbq + 16 * t);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lt + 32 * mbq + 16 * t + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dtv + 32 * mbq + 16 * t);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dtv + 32 * mbq + 16 * t + 4);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float pr[2], ds[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * e2 + u;   // query qb + 16 t + e
            const int r = 8 * t + e;
            const int qi = qb + 16 * t + e;
            const float nl = e < 4 ? l0[e & 3] : l1[e & 3];  // -LSE2 of the query
            const float dv = e < 4 ? d0[e & 3] : d1[e & 3];
            const float base = HAS_BIAS ? __builtin_fmaf(brow[(int64_t)min(qi, Nq - 1) * p.bias_sn], kLog2e, nl) : nl;
            pr[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c2, base));
            ds[u] = pr[u] * (pacc[r] - dv);
          }
          const bf16x2 pp = {(__bf16)pr[0], (__bf16)pr[1]};
          const bf16x2 dd = {(__bf16)ds[0], (__bf16)ds[1]};
          pb[t][e2] = __builtin_bit_cast(uint32_t, pp);
          db[t][e2] = __builtin_bit_cast(uint32_t, dd);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries (2 k-steps)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < kNcb; ++mb) {
          const int o = (2 * mbq + t) * G::kKBlock + 1024 * mb;
          const bf16x8 a_do = lds_read_tr_pair(dOt + tl0 + o, dOt + tl1 + o);
          const bf16x8 a_q = lds_read_tr_pair(Qt + tl0 + o, Qt + tl1 + o);
          dv_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_do, __builtin_bit_cast(bf16x8, pb[t]), dv_acc[mb], 0, 0, 0);
          dk_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_q, __builtin_bit_cast(bf16x8, db[t]), dk_acc[mb], 0, 0, 0);
        }
    }
    if (s + 1 < ns) {
      store_stats(buf ^ 1, nxt);
      wait_tiles();
    }
    __syncthreads();
  }

  // ---- epilogue: register r of block mb holds column 32 mb + 8 (r/4) + 4 hi + r%4;
  // keys at or past the key length get zero gradients
  if (my_k < Nk) {
    const float ks = my_k < kend ? p.scale : 0.f, vs = my_k < kend ? 1.f : 0.f;
    __bf16* dkrow = static_cast<__bf16*>(p.dk) + b * p.dk_sb + hk * p.dk_sh + (int64_t)my_k * p.dk_sn;
    __bf16* dvrow = static_cast<__bf16*>(p.dv) + b * p.dv_sb + hk * p.dv_sh + (int64_t)my_k * p.dv_sn;
#pragma unroll
    for (int mb = 0; mb < kNcb; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (__bf16)(dk_acc[mb][4 * g + e] * ks);
          wv[e] = (__bf16)(dv_acc[mb][4 * g + e] * vs);
        }
        *reinterpret_cast<bf16x4*>(dkrow + 32 * mb + 8 * g + 4 * hi) = wk;
        *reinterpret_cast<bf16x4*>(dvrow + 32 * mb + 8 * g + 4 * hi) = wv;
      }
  }
}

// ------------------------------------------------------------------- dQ
template <int D, int W, bool CAUSAL, bool HAS_BIAS, bool LOCAL>
__global__ __launch_bounds__(64 * W, 2) void bwd_dq_kernel(BwdParams p, TileMap tm) {
  using G = Geo<D, W>;
  constexpr int kBr = 32 * W;
  constexpr int kNkk = D / 16;
  constexpr int kNq = 2 * kNkk;  // MFMAs of one S^T (or dP^T) tile
  constexpr int kNcb = D / 32;
  constexpr int kStage = 2 * G::kKBytes;  // K tile, V tile
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  int b, h, qt, split;
  if (!decode_tile<false>(tm, p.B, p.H, b, h, qt, split)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int hk = h / p.head_group;
  const int Nq = p.Nq, Nk = p.Nk;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;
  const bool live = my_q < Nq;
  const float c2 = p.scale_log2;

  // Q and dO rows of this lane's query, resident: B operands of S^T and dP^T
  bf16x8 qf[kNkk], df[kNkk];
  float nl = -INFINITY, dval = 0.f;  // -LSE2 and D of this lane's query
  {
    const int qr = min(my_q, Nq - 1);
    const __bf16* qrow = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)qr * p.q_sn + 8 * hi;
    const __bf16* drow = static_cast<const __bf16*>(p.do_) + b * p.do_sb + h * p.do_sh + (int64_t)qr * p.do_sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kNkk; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk);
      df[kk] = *reinterpret_cast<const bf16x8*>(drow + 16 * kk);
    }
    if (live) {
      const int64_t row = ((int64_t)b * p.H + h) * Nq + my_q;
      nl = p.lse2[row];
      dval = p.dsum[row];
    }
  }

  // key range of this workgroup (as in the forward)
  int kend = Nk;
  if (p.kv_len != nullptr) kend = min(max(p.kv_len[b], 0), Nk);
  const int off = Nk - Nq + (LOCAL ? p.win_right : 0);
  const int off_l = Nk - Nq - p.win_left;
  const int qend = min(q0 + kBr, Nq);
  const int qmax_w = min(qw0 + 31, Nq - 1);
  int kstart = 0;
  if (LOCAL) kstart = max(q0 + off_l, 0) & ~(kBc - 1);
  int wg_keys = kend;
  if (CAUSAL) wg_keys = min(kend, qend + off);
  const int nt = wg_keys > kstart ? (wg_keys - kstart + kBc - 1) / kBc : 0;

  // LDS DMA sources as in the dK/dV kernel: row rrow0 + kRowStep * i, column rcol
  constexpr int kRowStep = dma_row_step<D, W>();
  const int rrow0 = rot_dma_row<D, W>(wave, lane, 0);
  const int rcol = k_dma_col<D, W>(wave, lane, 0);
  const int64_t ksn = p.k_sn * 2, vsn = p.v_sn * 2;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.k) + b * p.k_sb + hk * p.k_sh);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.v) + b * p.v_sb + hk * p.v_sh);
  // copy key tile j (keys kstart + 64 j ..) of K and V into buffer `buf`
  // (rows past the last key read the last key: masked to -inf, p = 0)
  auto issue = [&](int j, int buf) {
    const int kv0 = kstart + j * kBc;
    const int lim = Nk - 1 - kv0;
    uint8_t* st = smem + buf * kStage;
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i) {
      const int r = min(rrow0 + kRowStep * i, lim);
      dma16(kbase + kv0 * ksn, (uint32_t)(r * (int)ksn + rcol), st + 1024 * (wave + W * i));
      dma16(vbase + kv0 * vsn, (uint32_t)(r * (int)vsn + rcol), st + G::kKBytes + 1024 * (wave + W * i));
    }
  };
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 dq_acc[kNcb];
#pragma unroll
  for (int mb = 0; mb < kNcb; ++mb) dq_acc[mb] = f32x16{};
  const int rl0 = row_lane_offset(lane, G::kKBlock, 0), rl1 = row_lane_offset(lane, G::kKBlock, 1);
  const int tl0 = tr_lane_offset(lane, 0), tl1 = tr_lane_offset(lane, 1);
  const float* brow = nullptr;
  if (HAS_BIAS) brow = p.bias + b * p.bias_sb + h * p.bias_sh + (int64_t)min(my_q, Nq - 1) * p.bias_sn;

  if (nt > 0) {
    issue(0, 0);
    wait_tiles();
    __syncthreads();
  }
  for (int j = 0; j < nt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nt) issue(j + 1, buf ^ 1);
    const uint8_t* Kt = smem + buf * kStage;
    const uint8_t* Vt = Kt + G::kKBytes;
    const int kv0 = kstart + j * kBc;
    // S^T = K Q^T and dP^T = V dO^T: block bb = keys kv0 + 32 bb ..
    f32x16 sa[2] = {f32x16{}, f32x16{}}, da[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int i = 0; i < kNq; ++i) {
      const int o = (((i >> 1) & 1) ? rl1 : rl0) + (i & 1) * 2 * G::kKBlock + (i >> 1) * 512;
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Kt + o);
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vt + o);
      sa[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[i >> 1], sa[i & 1], 0, 0, 0);
      da[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, df[i >> 1], da[i & 1], 0, 0, 0);
    }
    // register r of block bb holds key kv0 + 32 bb + 16 (r/8) + 8 hi + (r%8)
    const bool need_mask = (kv0 + kBc > kend) || (CAUSAL && kv0 + kBc - 1 > qw0 + off) ||
                           (LOCAL && kv0 < qmax_w + off_l);
    // hidden scores become -inf in place (scale > 0: P = 0 below); only
    // tiles that cross the mask's edge or the key length take this branch
    if (need_mask) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
          if ((key >= kend) || (CAUSAL && key > my_q + off) || (LOCAL && key < my_q + off_l))
            sa[bb][r] = -INFINITY;
        }
    }
    u32x4 db[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float ds[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * r2 + u;
          const int key = kv0 + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
          const float base = HAS_BIAS ? __builtin_fmaf(brow[min(key, Nk - 1)], kLog2e, nl) : nl;
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[bb][r], c2, base));
          ds[u] = pr * (da[bb][r] - dval);
        }
        const bf16x2 dd = {(__bf16)ds[0], (__bf16)ds[1]};
        db[bb][r2 >> 2][r2 & 3] = __builtin_bit_cast(uint32_t, dd);
      }
    // dQ^T += K^T dS^T: 16-key group u = keys kv0 + 16 u ..
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mb = 0; mb < kNcb; ++mb) {
        const int o = u * G::kKBlock + 1024 * mb;
        const bf16x8 a = lds_read_tr_pair(Kt + tl0 + o, Kt + tl1 + o);
        dq_acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, db[u >> 1][u & 1]), dq_acc[mb], 0, 0, 0);
      }
    if (j + 1 < nt) wait_tiles();
    __syncthreads();
  }

  if (live) {
    __bf16* orow = static_cast<__bf16*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)my_q * p.dq_sn;
#pragma unroll
    for (int mb = 0; mb < kNcb; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 wq;
#pragma unroll
        for (int e = 0; e < 4; ++e) wq[e] = (__bf16)(dq_acc[mb][4 * g + e] * p.scale);
        *reinterpret_cast<bf16x4*>(orow + 32 * mb + 8 * g + 4 * hi) = wq;
      }
  }
}

template <typename Kern>
hipError_t set_lds(Kern kern, int bytes, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done = true;
  return e;
}

// wavefronts per workgroup of the dK/dV and dQ kernels (32 keys or rows each)
constexpr int kWkv = 4;
constexpr int kWq = 4;
// LDS requested per workgroup at d = 64 to hold two workgroups per CU
// instead of the three that registers and LDS would allow (the request is
// raised until only two fit in the CU's 160 KB): for dQ always, for dK/dV
// with a causal or window edge, whose deal groups heads for two per CU
// (dispatch_group). Measured A/B, c2 causal backward 172 -> 159 us, dense
// c2 263 -> 261 us (dK/dV capped on dense problems too: 264).
constexpr int kLdsTwoPerCu = 56 * 1024;

template <int D, bool CAUSAL, bool HAS_BIAS, bool LOCAL>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t s) {
  // dK / dV: key tiles of 32 * kWkv
  TileMap tk{};
  tk.n_qtiles = (p.Nk + 32 * kWkv - 1) / (32 * kWkv);
  tk.total = p.B * p.Hk * tk.n_qtiles;
  tk.per_xcd = (tk.total + 7) / 8;
  tk.group = CAUSAL ? dispatch_group(tk.n_qtiles, 2) : 1;  // two workgroups per CU
  if (tk.total > 0) {
    auto kern = bwd_dkdv_kernel<D, kWkv, CAUSAL, HAS_BIAS, LOCAL>;
    constexpr int lds0 = 2 * (2 * Geo<D, kWkv>::kKBytes + 2 * kBt * 4);
    constexpr int lds = (D == 64 && CAUSAL && lds0 < kLdsTwoPerCu) ? kLdsTwoPerCu : lds0;
    static bool done = false;
    hipError_t e = set_lds(kern, lds, done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(8 * tk.per_xcd), dim3(64 * kWkv), lds, s, p, tk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // dQ: query tiles of 32 * kWq
  TileMap tq{};
  tq.n_qtiles = (p.Nq + 32 * kWq - 1) / (32 * kWq);
  tq.total = p.B * p.H * tq.n_qtiles;
  tq.per_xcd = (tq.total + 7) / 8;
  tq.reverse_q = CAUSAL ? 1 : 0;
  tq.n_split = 1;
  tq.group = CAUSAL ? dispatch_group(tq.n_qtiles, 2) : 1;
  if (tq.total > 0) {
    auto kern = bwd_dq_kernel<D, kWq, CAUSAL, HAS_BIAS, LOCAL>;
    constexpr int lds0 = 2 * 2 * Geo<D, kWq>::kKBytes;
    constexpr int lds = (D == 64 && lds0 < kLdsTwoPerCu) ? kLdsTwoPerCu : lds0;
    static bool done = false;
    hipError_t e = set_lds(kern, lds, done);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(8 * tq.per_xcd), dim3(64 * kWq), lds, s, p, tq);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Launch dK/dV and dQ for the variants without a causal or window edge
// (bwd_bf16.hip) and for those with one (bwd_bf16_masked.hip); d is 64 or
// 128. The preprocess has run before either.
hipError_t launch_bwd_unmasked(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_bwd_masked(const BwdParams& p, int d, hipStream_t s);

}  // namespace attn
