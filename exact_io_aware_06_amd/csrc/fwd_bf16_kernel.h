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
//   * One workgroup = 8 wavefronts = 256 query rows of one (batch, head)
//     (4 wavefronts = 128 rows for d = 64 with a causal mask or a bias); each
//     wavefront owns 32 rows, so no cross-wave reduction of O is needed.
//   * Key/value tiles of 64 keys are copied global -> LDS directly
//     (global_load_lds_dwordx4, no staging registers), double buffered: the
//     loads of the next tiles are issued at the start of an iteration into
//     the buffers no wave reads any more and waited for just before the one
//     barrier that ends it.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys from LDS, B = 32 queries held in
//     VGPRs for the whole loop). In the 32x32 accumulator layout lane l holds
//     query l%32 and 16 of the 32 keys; the other 16 sit in lane l^32. A row
//     maximum is therefore in-lane max operations plus ONE cross-lane step
//     (v_permlane32_swap); the row sum needs no cross-lane step until the end.
//   * The rows of the K operand are fed in a fixed permutation (bits 2 and 3
//     of the row index swapped) so that the accumulator registers 8t..8t+7 of
//     every lane hold 8 consecutive keys. They are converted to bf16 in place
//     and used directly as the B operand of O^T += V^T P^T, with no shuffle.
//   * The A operand of that product (8 consecutive keys of one V column per
//     lane) is read from the row-major V tile with two ds_read_b64_tr_b16:
//     within a group of 16 lanes, lane i receives element i%4 of the 8-byte
//     chunks addressed by lanes 4e + i/4 (e = 0..3), so 16 lanes that address
//     4 key rows x 16 columns come back holding one column of 4 keys each.
//   * In LDS, K rows are interleaved in blocks of 16 (16-byte chunk c of row
//     r at slot 16c + r) and V rows in blocks of 4 (slot 4c + r), so the rows
//     one MFMA operand reads fall in distinct banks while every read address
//     is a per-lane base plus an immediate offset.
//   * The running maximum is replaced by a reference point R per row: any R
//     gives the same result in exact arithmetic ("Understanding FlashAttention
//     Pt 1", section 2.2: the maximum is only a change of reference), as long
//     as no probability 2^(s - R) overflows. R starts at the exact maximum of
//     the first tile. Each later tile is exponentiated against R directly,
//     without computing its maximum; before the O^T product consumes the
//     probabilities, the per-lane sum of the tile's probabilities (an upper
//     bound of each of them) is checked against 2^32. Only if it is larger
//     (or not finite, or the row has no reference yet) does the wave compute
//     the tile's exact maximum, move R up to it, rescale O and the
//     denominator by 2^(R_old - R_new) and exponentiate the tile again (the
//     conditional rescaling of "FlashAttention, Explained", section 22, made
//     rare). Probabilities therefore stay below 2^32 and far from overflow.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fwd_params.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBc = 64;           // keys per tile
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kBig = 4294967296.0f;  // 2^32: bound on a lane's probability sum per tile
constexpr int kPf = 4;            // MFMA operands read ahead from LDS

// W = wavefronts per workgroup (8, or 4 where finer workgroups balance
// uneven work better); each wavefront owns 32 query rows.
template <int D, int W>
struct Geo {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kBr = 32 * W;                  // query rows per workgroup
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kKBlock = 16 * kChunks * 16;   // 16 K rows, chunk-interleaved
  static constexpr int kVBlock = 4 * kChunks * 16;    // 4 V rows, chunk-interleaved
  static constexpr int kKBytes = kBc * D * 2;
  static constexpr int kVBytes = kBc * D * 2;
  static constexpr int kSmem = 2 * (kKBytes + kVBytes);
  static constexpr int kDma = kKBytes / 1024;         // 1 KB DMA instructions per tile (K or V)
  static constexpr int kDmaPerWave = kDma / W;
  // Bias tiles staged in LDS (d = 64 biased kernels): each wave copies the
  // 32 x 64 fp32 bias block of its own rows, 8 KB.
  static constexpr int kBiasWave = 32 * kBc * 4;
  static constexpr int kBiasBytes = W * kBiasWave;
  static constexpr int kNkk = D / 16;                 // k-steps of QK^T
  static constexpr int kNcb = D / 32;                 // 32-wide output column blocks
};

// Row permutation of the K operand: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Source of the 16 bytes that `lane` of wave `wave` fetches in DMA
// instruction i of a tile (instruction n of a tile is issued by wave n % W
// and fills LDS bytes [1024 n, 1024 n + 1024)): key row within the tile and
// byte column within the row. K tiles are chunk-interleaved in blocks of 16
// rows with the rows permuted (perm_row), V tiles in blocks of 4.
template <int D, int W>
__device__ __forceinline__ int k_dma_key(int wave, int lane, int i) {
  const int a = 1024 * (wave + W * i) + 16 * lane;
  constexpr int blk = 16 * (D / 8) * 16;
  const int ks = (a % blk) / 16;
  return perm_row(16 * (a / blk) + ks % 16);
}
template <int D, int W>
__device__ __forceinline__ int k_dma_col(int wave, int lane, int i) {
  const int a = 1024 * (wave + W * i) + 16 * lane;
  return 16 * ((a % (16 * (D / 8) * 16)) / 256);
}
template <int D, int W>
__device__ __forceinline__ int v_dma_key(int wave, int lane, int i) {
  const int a = 1024 * (wave + W * i) + 16 * lane;
  constexpr int blk = 4 * (D / 8) * 16;
  return 4 * (a / blk) + ((a % blk) / 16) % 4;
}
template <int D, int W>
__device__ __forceinline__ int v_dma_col(int wave, int lane, int i) {
  const int a = 1024 * (wave + W * i) + 16 * lane;
  return 16 * ((a % (4 * (D / 8) * 16)) / 64);
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

// A copy of a lane-constant value that the compiler must recompute where it
// is used: at 256 registers, values derived from the lane index that are
// hoisted out of a loop get spilled and reloaded every iteration, while
// recomputing them costs one or two vector instructions.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A pointer that every lane holds, moved to scalar registers (the copy
// instructions take their base address from an SGPR pair; the compiler may
// keep a value derived from per-lane data in VGPRs even when it is uniform).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Two LDS transpose reads (4 keys each) concatenated into one MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint8_t* p0, const uint8_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<uint8_t*>(p0)));
  const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<uint8_t*>(p1)));
  const s16x8 v = __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// 16 bytes from global memory (tile + off) straight into LDS at
// lds_base + 16 * lane. tile and lds_base are uniform. Written as inline asm
// so that the compiler does not treat every later LDS read as a possible
// alias of the copy and wait for it (vmcnt(0)), nor drain the LDS read queue
// (lgkmcnt(0)) after issuing it: the kernel orders the copies itself with
// s_waitcnt vmcnt and a barrier before any wave reads the buffer.
// The compiler's hazard pass cannot see that the asm is a vector-memory
// load reading M0 and two SGPRs, so the asm carries its own wait states:
// GFX9-family parts need 1 after a scalar write of M0 before an LDS-DMA load,
// and 5 after a vector-ALU write of an SGPR (e.g. v_readlane restoring a
// spilled address register) before a vector-memory instruction reads it.
// s_nop 4 gives 5 whatever the compiler placed before the copy.
__device__ __forceinline__ void dma16(const uint8_t* tile, uint32_t off, uint8_t* lds_base) {
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_u8*)lds_base;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(tile), "{m0}"(lds));
}
// The same copy with the non-temporal hint, for data read once (the K/V
// tiles of a key-split launch: each key range is read by one workgroup):
// measured 8-10% faster on the decoding workloads (6.4 TB/s at batch 8,
// 16K keys) than the default policy.
__device__ __forceinline__ void dma16_nt(const uint8_t* tile, uint32_t off, uint8_t* lds_base) {
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_u8*)lds_base;
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(tile), "{m0}"(lds));
}

// Work item `logical` as (tile, flat head index). group <= 1: tile fastest,
// then head. group > 1: heads are dealt in groups of `group` (the last
// group may be smaller) and within a group the tile is the slow index, so
// with the longest tiles first (causal) the longest tiles of every head of
// the group start before any shorter one, while the workgroups resident on
// an XCD still read about `group` heads' K/V (a greedy dispatch of
// longest-first work, as in list scheduling).
__device__ __forceinline__ void split_logical(int logical, int n_tiles, int n_heads, int group,
                                              int& tile, int& hb) {
  if (group <= 1) {
    tile = logical % n_tiles;
    hb = logical / n_tiles;
    return;
  }
  const int g0 = logical / (group * n_tiles) * group;
  const int gs = min(group, n_heads - g0);
  const int within = logical - g0 * n_tiles;
  tile = within / gs;
  hb = g0 + within % gs;
}

template <bool SPLIT, bool VARLEN = false>
__device__ __forceinline__ bool decode_tile(const TileMap& tm, int B, int H,
                                            int& b, int& h, int& qt, int& split) {
  const int w = blockIdx.x;
  int rest;
  int qi;
  split = 0;
  if (VARLEN) {
    // (batch, head) groups dealt round-robin over the 8 XCDs (workgroup w
    // runs on XCD w % 8): one group's query tiles stay on one XCD and share
    // its L2, and sequences of very different lengths spread evenly
    const int x = w & 7, j = w >> 3;
    const int g = (j / tm.n_qtiles) * 8 + x;
    if (g >= B * H) return false;
    qi = j % tm.n_qtiles;
    h = g % H;
    b = g / H;
    qt = tm.reverse_q ? (tm.n_qtiles - 1 - qi) : qi;
    return true;
  }
  const int logical = (w & 7) * tm.per_xcd + (w >> 3);
  if (logical >= tm.total) return false;
  if (SPLIT) {
    // query tile fastest (they read the same key range), then the split
    qi = logical % tm.n_qtiles;
    rest = logical / tm.n_qtiles;
    split = rest % tm.n_split;
    rest /= tm.n_split;
    h = rest % H;
    b = rest / H;
  } else if (tm.batch_inner) {
    b = logical % B;
    rest = logical / B;
    qi = rest % tm.n_qtiles;
    h = rest / tm.n_qtiles;
  } else {
    split_logical(logical, tm.n_qtiles, B * H, tm.group, qi, rest);
    h = rest % H;
    b = rest / H;
  }
  qt = tm.reverse_q ? (tm.n_qtiles - 1 - qi) : qi;
  return true;
}

// SPLIT: one split of the keys per workgroup, partial results to the
// workspace (p.n_split > 1); otherwise all keys, results to o / lse.
// CAUSAL: keys j > i + (Nk - Nq) hidden from query i, or, with LOCAL, keys
// outside the window [i + (Nk - Nq) - win_left, i + (Nk - Nq) + win_right].
// VARLEN: the batch index is a packed sequence of its own length (rows and
// keys from the cumulative offsets p.cu_q / p.cu_k).
template <int D, int W, bool CAUSAL, bool HAS_BIAS, bool SPLIT, bool LOCAL, bool VARLEN = false>
__global__ __launch_bounds__(64 * W, 2) void fwd_bf16_kernel(FwdParams p, TileMap tm) {
  static_assert(CAUSAL || !LOCAL, "a window is a two-sided causal mask");
  static_assert(!VARLEN || (!HAS_BIAS && !SPLIT), "packed sequences take neither a bias nor a split");
  using G = Geo<D, W>;
  constexpr int kWaves = G::kWaves;
  constexpr int kBr = G::kBr;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  // packed: the query heads of one key/value head share the workgroup's rows
  const bool packed = SPLIT && p.pack > 1;
  int b, h, qt, split;
  // Paired batches (d = 64 with a batch-broadcast bias and key lengths,
  // tm.pairs > 0): the batches are ranked by key length (longest first) and
  // the workgroup of pair r runs two items of one (head, query tile): the
  // batch of rank r, then that of rank B-1-r, so every workgroup does about
  // the same work whatever the lengths (a long batch with a short one), and
  // the batches of one bias tile run together. Without pairing, items of
  // very different lengths share the CUs and the last CUs to finish hold the
  // whole launch (list-scheduling model of the padded-bias workload: 1.5x
  // the balanced time).
  constexpr bool kPairable = D == 64 && HAS_BIAS && !CAUSAL && !SPLIT && !VARLEN;
  int b_next = -1;
  if (kPairable && tm.pairs > 0) {
    const int w = blockIdx.x;
    const int logical = (w & 7) * tm.per_xcd + (w >> 3);
    if (logical >= tm.total) return;
    const int pr = logical % tm.pairs;
    const int rest = logical / tm.pairs;
    qt = rest % tm.n_qtiles;
    h = rest / tm.n_qtiles;
    split = 0;
    // rank of batch `lane` (B <= 64): longer key lengths first, ties by index
    const int ln = threadIdx.x & 63;
    const int kl = ln < p.B ? min(max(p.kv_len[ln], 0), p.Nk) : -1;
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
      const int kj = __builtin_amdgcn_readlane(kl, j);
      rank += (kj > kl || (kj == kl && j < ln)) ? 1 : 0;
    }
    auto batch_of = [&](int r) {
      return (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(ln < p.B && rank == r));
    };
    b = batch_of(pr);
    if (p.B - 1 - pr != pr) b_next = batch_of(p.B - 1 - pr);
  } else if (!decode_tile<SPLIT, VARLEN>(tm, p.B, packed ? p.Hk : p.H, b, h, qt, split)) {
    return;
  }
  if (VARLEN && tm.rank_seq) {
    // packed sequences: decode_tile's sequence index is a rank; the
    // sequences are ranked by query x key length (ties by index), so the
    // longest ones start first and the shorter ones fill in behind them
    // (a list-scheduling model of the packed workload: 1.12x the ideal
    // time in sequence order, 1.03x longest first)
    const int ln = threadIdx.x & 63;
    float wl = -1.f;
    if (ln < p.B) {
      const int a0 = min(max(p.cu_q[ln], 0), p.Nq), a1 = min(max(p.cu_q[ln + 1], a0), p.Nq);
      const int c0 = min(max(p.cu_k[ln], 0), p.Nk), c1 = min(max(p.cu_k[ln + 1], c0), p.Nk);
      wl = (float)(a1 - a0) * (float)(c1 - c0);
    }
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), j));
      rank += (wj > wl || (wj == wl && j < ln)) ? 1 : 0;
    }
    b = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(ln < p.B && rank == b));
  }

  for (int item = 0; item < (kPairable ? 2 : 1); ++item) {
  if (item == 1) {
    if (b_next < 0) break;
    b = b_next;
    // the first item's last reads of the K/V and bias buffers are done
    // before the second item's prologue copies into them
    __syncthreads();
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in SGPRs
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int hk = packed ? h : h / p.head_group;

  // Rows [0, Nq) and keys [0, NkAll) of this (batch, head); packed
  // sequences start at row q_lo / key k_lo of the packed tensors, with the
  // offsets clamped into the tensors whatever the offset arrays hold.
  int Nq = p.Nq, NkAll = p.Nk;
  int64_t q_lo = 0, k_lo = 0;
  if (VARLEN) {
    const int a0 = min(max(p.cu_q[b], 0), p.Nq), a1 = min(max(p.cu_q[b + 1], a0), p.Nq);
    const int c0 = min(max(p.cu_k[b], 0), p.Nk), c1 = min(max(p.cu_k[b + 1], c0), p.Nk);
    q_lo = a0;
    Nq = a1 - a0;
    k_lo = c0;
    NkAll = c1 - c0;
    if (qt * kBr >= Nq) return;  // past this sequence's rows (the grid covers the longest)
  }
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;   // this lane's row of the workgroup's row space

  // Row r of the row space is query r of head h, or, packed, query r % Nq
  // of query head h * pack + r / Nq. row_i: this lane's query index;
  // qmin_w / qmax_w: the smallest / largest query index of the wave's rows;
  // qbeg / qend: the smallest / one past the largest of the workgroup's rows
  // (they bound the causal mask and the window).
  int row_h = h, row_i = my_q, nrows = Nq, qmin_w = qw0, qend = min(q0 + kBr, Nq);
  int qmax_w = min(qw0 + 31, Nq - 1), qbeg = q0;
  if (packed) {
    nrows = p.pack * Nq;
    const int rr = min(my_q, nrows - 1);
    row_h = h * p.pack + rr / Nq;
    row_i = rr % Nq;
    const int wl = min(qw0 + 31, nrows - 1), gl = min(q0 + kBr - 1, nrows - 1);
    qmin_w = (qw0 / Nq == wl / Nq) ? qw0 % Nq : 0;
    qmax_w = (qw0 / Nq == wl / Nq) ? wl % Nq : Nq - 1;
    qend = (q0 / Nq == gl / Nq) ? gl % Nq + 1 : Nq;
    qbeg = (q0 / Nq == gl / Nq) ? q0 % Nq : 0;
  }
  const bool row_live = my_q < nrows;
  const __bf16* qg = static_cast<const __bf16*>(p.q) + (VARLEN ? q_lo * p.q_sn : b * p.q_sb) +
                     row_h * p.q_sh;

  // Key range. Split over keys: this workgroup covers keys [s * kv_split,
  // (s + 1) * kv_split) of its rows. Window: whole tiles before the window
  // of its first row are skipped. kbeg is the first key it reads; key
  // indices below are relative to kbeg (the K/V and bias base addresses,
  // the key count and the mask offsets are shifted by it).
  int kbeg = SPLIT ? split * p.kv_split : 0;
  if (LOCAL) kbeg = max(kbeg, max(qbeg + NkAll - Nq - p.win_left, 0) & ~(kBc - 1));
  const __bf16* kgp = static_cast<const __bf16*>(p.k) + (VARLEN ? k_lo * p.k_sn : b * p.k_sb) +
                      hk * p.k_sh + (int64_t)kbeg * p.k_sn;
  const __bf16* vgp = static_cast<const __bf16*>(p.v) + (VARLEN ? k_lo * p.v_sn : b * p.v_sb) +
                      hk * p.v_sh + (int64_t)kbeg * p.v_sn;
  const int Nk = NkAll - kbeg;  // keys from kbeg on
  // causal alignment: key j hidden from query i when j > i + off (and, with
  // a window, when j < i + off_l)
  const int off = NkAll - Nq - kbeg + (LOCAL ? p.win_right : 0);
  const int off_l = NkAll - Nq - kbeg - p.win_left;

  int kend = Nk;
  if (p.kv_len != nullptr) kend = min(max(p.kv_len[b] - kbeg, 0), Nk);
  if (SPLIT) kend = min(kend, LOCAL ? (split + 1) * p.kv_split - kbeg : p.kv_split);
  int wg_keys = kend;
  if (CAUSAL) wg_keys = min(kend, qend + off);
  wg_keys = max(wg_keys, 0);
  const int nt = (wg_keys + kBc - 1) / kBc;
  // Window without a key split: the key tiles are visited in a rotated
  // order, step j taking the tile whose absolute index (counted from key 0)
  // is congruent to j modulo nt, wrapping at the end of the range. Every
  // workgroup with a whole window covers the same number of tiles, so the
  // query tiles of one head that run side by side on an XCD read each key
  // tile at the same step and all but the first copy come from L2 (in
  // ascending order the band of 32 neighbouring query tiles spans more than
  // an XCD's L2 between the first and the last read of a tile). Not done
  // when a tile runs past the last key: such a tile's copy offsets are
  // clamped in place and must not be followed by whole tiles.
  int rot = 0;
  if constexpr (LOCAL && !SPLIT) {
    if (nt > 0 && nt * kBc <= Nk) rot = (nt - (kbeg / kBc) % nt) % nt;
  }
  auto ktile = [&](int j) {
    const int x = j + rot;
    return x >= nt ? x - nt : x;
  };

  // ---- Q as the B operand, resident for the whole loop: lane holds query
  // row_i, elements [16kk + 8hi, 16kk + 8hi + 8).
  bf16x8 qf[G::kNkk];
  if (row_live) {
    const __bf16* qrow = qg + (int64_t)row_i * p.q_sn + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < G::kNkk; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < G::kNkk; ++kk)
      qf[kk] = bf16x8{};
  }

  // ---- tile loads: global memory -> LDS directly (global_load_lds_dwordx4),
  // no registers involved. One such instruction writes 1 KB of LDS, lane l
  // at byte 16l; which global 16 bytes a lane fetches is free, so the LDS
  // layouts below are produced by choosing each lane's source address.
  //   K tile: blocks of 16 rows; inside a block, 16-byte slot
  //     (chunk * 16 + row % 16). LDS row R holds key perm_row(R) (low 5 bits).
  //   V tile: blocks of 4 rows; inside a block, slot (chunk * 4 + row % 4).
  // DMA instruction n (0 <= n < kDma) of a tile is issued by wave n % kWaves.
  // Rows past the last key are read from the last key row instead (always a
  // valid address, finite data): their scores are masked to -inf, so their
  // probabilities are exactly 0 and they contribute nothing.
  // Each lane's source offset inside a full tile is fixed: a 32-bit byte
  // offset added to the tile's base address, which is uniform (SGPRs).
  uint32_t koff[G::kDmaPerWave], voff[G::kDmaPerWave];
  const int64_t ksn = p.k_sn * 2, vsn = p.v_sn * 2;   // row strides in bytes
#pragma unroll
  for (int i = 0; i < G::kDmaPerWave; ++i) {
    koff[i] = (uint32_t)(k_dma_key<D, W>(wave, lane, i) * (int)ksn + k_dma_col<D, W>(wave, lane, i));
    voff[i] = (uint32_t)(v_dma_key<D, W>(wave, lane, i) * (int)vsn + v_dma_col<D, W>(wave, lane, i));
  }
  const int last_key = Nk - 1;
  uint8_t* const kbuf = smem;                  // K tile t in buffer t % 2
  uint8_t* const vbuf = smem + 2 * G::kKBytes; // V tile t in buffer t % 2
  const uint8_t* const kbase = reinterpret_cast<const uint8_t*>(kgp);
  const uint8_t* const vbase = reinterpret_cast<const uint8_t*>(vgp);
  // Base address of key tile j (uniform). A tile that runs past the last key
  // is the last tile of its kind ever loaded (later loads only fetch it
  // again), so its clamped offsets simply replace the fixed ones.
  auto prep_k = [&](int j) {
    const int kv0 = ktile(j) * kBc;
    if (kv0 + kBc > Nk) {
#pragma unroll
      for (int i = 0; i < G::kDmaPerWave; ++i)
        koff[i] = (uint32_t)(min(k_dma_key<D, W>(wave, lane, i), last_key - kv0) * (int)ksn +
                             k_dma_col<D, W>(wave, lane, i));
    }
    return kbase + kv0 * ksn;
  };
  auto prep_v = [&](int j) {
    const int kv0 = ktile(j) * kBc;
    if (kv0 + kBc > Nk) {
#pragma unroll
      for (int i = 0; i < G::kDmaPerWave; ++i)
        voff[i] = (uint32_t)(min(v_dma_key<D, W>(wave, lane, i), last_key - kv0) * (int)vsn +
                             v_dma_col<D, W>(wave, lane, i));
    }
    return vbase + kv0 * vsn;
  };
  // DMA instruction i of this wave for a K (V) tile at `tile` into buffer `dst`
  auto dma_k = [&](const uint8_t* tile, uint8_t* dst, int i) {
    if constexpr (SPLIT) dma16_nt(tile, koff[i], dst + 1024 * (wave + kWaves * i));
    else dma16(tile, koff[i], dst + 1024 * (wave + kWaves * i));
  };
  auto dma_v = [&](const uint8_t* tile, uint8_t* dst, int i) {
    if constexpr (SPLIT) dma16_nt(tile, voff[i], dst + 1024 * (wave + kWaves * i));
    else dma16(tile, voff[i], dst + 1024 * (wave + kWaves * i));
  };
  auto load_k = [&](int j) {
    const uint8_t* t = prep_k(j);
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i) dma_k(t, kbuf + (j & 1) * G::kKBytes, i);
  };
  auto load_v = [&](int j) {
    const uint8_t* t = prep_v(j);
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i) dma_v(t, vbuf + (j & 1) * G::kVBytes, i);
  };
  // the DMA writes count as outstanding vector-memory loads
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // ---- MFMA operand addressing (per lane, fixed).
  // K: lane reads row 32bb + l32, 16-byte chunk 2kk + hi:
  //   32bb*... + (l32/16) * kKBlock + (2kk + hi) * 256 + (l32 % 16) * 16.
  const uint8_t* const klane = kbuf + (l32 >> 4) * G::kKBlock + hi * 256 + (l32 & 15) * 16;
  // V^T: in its 16-lane group, lane i reads key row 4s + i/4 (+ 8hi +
  // block/half offsets), 8-byte chunk 8cb + 4*(l32/16) + i%4, i.e. 16-byte
  // chunk 4cb + 2*(l32/16) + (i/2)%2, half i%2, in 4-row block row/4.
  const int gi = l32 & 15;
  const uint8_t* const vlane = vbuf + 2 * hi * G::kVBlock + 128 * (l32 >> 4) +
                               64 * ((gi >> 1) & 1) + 16 * (gi >> 2) + 8 * (gi & 1);
  constexpr int kNq = 2 * G::kNkk;   // MFMAs of one S^T tile
  constexpr int kNv = 4 * G::kNcb;   // MFMAs of one O^T update
  // MFMA i of S^T: k-step i/2 of key block i%2
  auto kfrag = [&](const uint8_t* kb, int i) {
    return *reinterpret_cast<const bf16x8*>(kb + (i & 1) * 2 * G::kKBlock + (i >> 1) * 512);
  };
  // MFMA i of O^T: column block i % kNcb, 16-key group u = i / kNcb (key
  // block u/2, half u%2; rows 16u + 8hi + 4s + [0, 4)); consecutive MFMAs
  // update different column blocks so no MFMA waits for the previous one
  auto vfrag = [&](const uint8_t* vb, int i) {
    const uint8_t* p0 = vb + 4 * (i / G::kNcb) * G::kVBlock + 256 * (i % G::kNcb);
    return lds_read_tr_pair(p0, p0 + G::kVBlock);
  };

  // ---- running state of this lane's query row
  f32x16 oacc[G::kNcb];
#pragma unroll
  for (int cb = 0; cb < G::kNcb; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;  // reference R of this lane's row, base-2 units (-inf: none yet)
  float l_run = 0.f;        // this lane's share of the running denominator
  const float c2 = p.scale_log2;

  const float* brow = nullptr;
  if (HAS_BIAS) {
    const int qrow = min(row_i, Nq - 1);
    brow = p.bias + b * p.bias_sb + row_h * p.bias_sh + (int64_t)qrow * p.bias_sn + kbeg + 8 * hi;
  }

  // ---- bias tiles through LDS (d = 64, host-checked layout, p.bias_dma):
  // each wave copies the bias block of its own 32 rows into its own 8 KB of
  // LDS (no other wave reads it, so no barrier is involved). The block of
  // tile t+1 is copied right after the wave has read that of tile t (in
  // iteration t-1, after that iteration's K/V copies). Vector memory
  // operations complete in issue order, so that iteration ends with
  // vmcnt(8) (the block may still be in flight; every K/V copy has landed),
  // and iteration t waits vmcnt(kNdma) before reading it (its own K/V
  // copies, issued later, may still be in flight): each block has about a
  // full iteration to arrive instead of being loaded where it is used.
  // LDS layout of a wave's block: 16-byte chunk kc (keys 4kc..4kc+3) of
  // row r at slot 16 r + (kc ^ (r % 16)), so the 16 lanes of one row copy
  // 256 contiguous bytes and the reads of 16 rows hit 16 different banks.
  constexpr bool kBiasLds = HAS_BIAS && D == 64;
  const bool bias_dma = kBiasLds && p.bias_dma;
  uint8_t* const bias_lds = smem + G::kSmem + wave * G::kBiasWave;
  const uint8_t* bias_wave = nullptr;  // row min(qw0, Nq-1) of the bias, key kbeg
  int bias_rmax = 0;                   // rows of this wave that exist, minus 1
  uint32_t boff[kBiasLds ? 8 : 1];     // lane's source offsets for a full tile
  if constexpr (kBiasLds) {
    if (bias_dma) {
      const int rbase = min(qw0, Nq - 1);
      bias_rmax = Nq - 1 - rbase;
      bias_wave = reinterpret_cast<const uint8_t*>(p.bias + b * p.bias_sb + row_h * p.bias_sh +
                                                   (int64_t)rbase * p.bias_sn + kbeg);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int kc = (lane & 15) ^ (r & 15);
        boff[i] = (uint32_t)(min(r, bias_rmax) * (int)(p.bias_sn * 4) + 16 * kc);
      }
    }
  }
  // copy the block of tile j (the last tile's chunks past the last key read
  // the row's last four keys instead: finite, and masked)
  auto dma_bias = [&](int j) {
    if constexpr (kBiasLds) {
      const int kv0 = ktile(j) * kBc;
      const uint8_t* t = uniform_ptr(bias_wave + 4 * kv0);
      if (kv0 + kBc <= Nk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma16(t, boff[i], bias_lds + 1024 * i);
      } else {
        const int ln = fresh(lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 4 * i + (ln >> 4);
          const int kc = (ln & 15) ^ (r & 15);
          const int key = min(4 * kc, Nk - 4 - kv0);
          dma16(t, (uint32_t)(min(r, bias_rmax) * (int)(p.bias_sn * 4) + 4 * key),
                bias_lds + 1024 * i);
        }
      }
    }
  };

  // Bias and masks of tile j. Register r of block bb holds key
  // kv0 + 32bb + 16(r/8) + 8hi + (r%8). With a bias the scores become
  // scale * qk + bias in natural units (one FMA); the exponent's FMA turns
  // them into base 2 (without one, the raw qk goes there with scale * log2 e).
  auto mask_bias = [&](int j, f32x16 (&s)[2]) {
    const int kv0 = ktile(j) * kBc;
    if (HAS_BIAS) {
      f32x16 bia[2];
      const bool fullb = p.bias_vec && kv0 + kBc <= Nk;
      if (bias_dma) {
        // this wave's block of tile j, from LDS (see dma_bias): chunk
        // 8bb + 4s2 + 2hi + half of row l32
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G::kDmaPerWave) : "memory");
        const uint8_t* rowp = bias_lds + 256 * l32;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int kc = 8 * bb + 4 * s2 + 2 * hi + half;
              const f32x4 x = *reinterpret_cast<const f32x4*>(rowp + 16 * (kc ^ (l32 & 15)));
#pragma unroll
              for (int e = 0; e < 4; ++e) bia[bb][8 * s2 + 4 * half + e] = x[e];
            }
      } else {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float* src = brow + kv0 + 32 * bb + 16 * s2;
          if (fullb) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bia[bb][8 * s2 + e] = x0[e];
              bia[bb][8 * s2 + 4 + e] = x1[e];
            }
          } else {
            const int k0 = kv0 + 32 * bb + 16 * s2 + 8 * hi;
#pragma unroll
            for (int e = 0; e < 8; ++e) bia[bb][8 * s2 + e] = (k0 + e < Nk) ? src[e] : 0.f;
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[bb][r] = __builtin_fmaf(s[bb][r], p.scale, bia[bb][r]);
      if (bias_dma && j + 1 < nt) {
        // the block of tile j+1 replaces it once this wave's reads are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        dma_bias(j + 1);
      }
    }
    const bool need_mask = (kv0 + kBc > kend) || (CAUSAL && kv0 + kBc - 1 > qmin_w + off) ||
                           (LOCAL && kv0 < qmax_w + off_l);
    if (need_mask) {
      const int lim_c = row_i + off;    // last key this query may see (causal)
      const int lim_l = row_i + off_l;  // first key it may see (window)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
          const bool hide = (key >= kend) || (CAUSAL && key > lim_c) || (LOCAL && key < lim_l);
          if (hide) s[bb][r] = -INFINITY;
        }
    }
  };

  // The softmax of one tile is split into slices that are placed between
  // MFMAs of the other product, so the vector ALUs and the matrix pipe work
  // at the same time within one wavefront. Slices are straight-line VALU
  // code; sched_barrier fences pin each slice after its MFMA.
  //
  // Exact maximum of a score tile for this lane's row, in base-2 units (the
  // lane pair l, l^32 holds the row's 64 keys). Used for the first tile and
  // on the rare path only.
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float m = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, s[bb][r]);
    m = lane_pair_max(m);
    return m * (HAS_BIAS ? kLog2e : c2);
  };
  // Exponential slice: scores 2i and 2i+1 of the tile (block i/8, registers
  // 2(i%8), 2(i%8)+1) -> probabilities, their sum, and one packed bf16 pair
  // of the P^T operand (registers 8t..8t+7 of block bb = keys
  // 32bb + 16t + 8hi + [0, 8)).
  auto exp_slice = [&](const f32x16 (&s)[2], u32x4 (&pw)[2][2], float m_use, float& rs, int i) {
    const int bb = i >> 3, r = 2 * (i & 7);
    float x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float t = __builtin_fmaf(s[bb][r + e], HAS_BIAS ? kLog2e : c2, -m_use);
      x[e] = __builtin_amdgcn_exp2f(t);
      rs += x[e];
    }
    const bf16x2 v = {(__bf16)x[0], (__bf16)x[1]};
    uint32_t w = __builtin_bit_cast(uint32_t, v);
    // keep the slice here: without a use in this block the compiler sinks
    // the exponentials down to the PV MFMAs that consume them
    asm volatile("" : "+v"(w), "+v"(rs));
    pw[bb][r >> 3][(r & 7) >> 1] = w;
  };

  // ---- software pipeline over key tiles (per wavefront):
  //   phase A of iteration j: S_{j+1} = K_{j+1} Q^T on the matrix pipe,
  //       exponentials/sums/bf16 packing of the second half (keys 32..63) of
  //       tile j on the vector ALUs;
  //   then the overflow check of tile j over both halves (rarely: its exact
  //       maximum, the move of the reference and all its exponentials
  //       again), masks of tile j+1;
  //   phase B: O += V_j P_j on the matrix pipe; beside its second half (which
  //       reads only the second half of P_j) the exponentials of the first
  //       half (keys 0..31) of tile j+1, into the registers of P_j's first
  //       half, against the reference as it stands after tile j.
  // The vector work of a tile is thus split between both phases, and the
  // check of tile j+1 still sees all of its probabilities before any of
  // them is consumed.
  // The LDS holds K_{j+1} and V_j during iteration j; K_{j+2} and V_{j+1}
  // are loaded meanwhile and written to the buffers of K_j and V_{j-1},
  // which no wave reads any more (one barrier per iteration).
  constexpr int kSlices = 16;       // exponential slices per tile (two scores each)
  // slices of the first 32-key half computed ahead in the previous phase B:
  // 8 without a mask edge or bias; with one, all slices stay in phase A
  // (measured: the split gains 1-3% on unmasked problems and loses 0.2-2%
  // with a causal or window edge, whose extra registers it would spill)
  constexpr int kPre = (CAUSAL || HAS_BIAS) ? 0 : kSlices / 2;
  constexpr int kSlicesA = kSlices - kPre;  // slices computed in phase A
  constexpr int kNdma = 2 * G::kDmaPerWave;  // K then V DMA instructions per wave and tile
  auto phase_a = [&](auto with_qk, const uint8_t* kb, const f32x16 (&sc)[2], f32x16 (&sn)[2],
                     u32x4 (&pb)[2][2], float m_use, auto&& dma) {
    float rs = 0.f;
    // Wave priority: 1 in phase A, 0 in phase B. The two waves of a SIMD start
    // a tile together; the one that reaches phase B first (MFMAs only) then
    // yields issue slots to the other, still in its vector-heavy phase A, so
    // both arrive at the barrier closer together.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (decltype(with_qk)::value) {
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      bf16x8 kf[kPf];
#pragma unroll
      for (int i = 0; i < kPf; ++i) kf[i] = kfrag(kb, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kNq; ++i) {
        sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % kPf], qf[i >> 1], sn[i & 1], 0, 0, 0);
        if (i + kPf < kNq) kf[i % kPf] = kfrag(kb, i + kPf);
        dma(i);
#pragma unroll
        for (int k = (kSlicesA * i) / kNq; k < (kSlicesA * (i + 1)) / kNq; ++k)
          exp_slice(sc, pb, m_use, rs, kPre + k);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int k = kPre; k < kSlices; ++k) exp_slice(sc, pb, m_use, rs, k);
    }
    return rs;
  };
  // with_next: also the first-half exponentials of the next tile (sn) into
  // pb[0], their sum into rs_next
  auto phase_b = [&](auto with_next, const uint8_t* vb, u32x4 (&pb)[2][2], const f32x16 (&sn)[2],
                     float m_use, float& rs_next) {
    __builtin_amdgcn_s_setprio(0);
    bf16x8 vf[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) vf[i] = vfrag(vb, i);
    __builtin_amdgcn_sched_barrier(0);
    // the kPre slices go beside the last MFMAs, 16 / kNv per MFMA from
    // MFMA kB0 on; slice k writes 16-key group k / 4 of pb, which MFMAs
    // [kNcb * (k / 4), kNcb * (k / 4 + 1)) read: every one of them precedes
    // the slice when kPre <= 12
    constexpr int kPer = kSlices / kNv;
    constexpr int kB0 = kNv - kPre / kPer;
    static_assert(kPre % kPer == 0 && kPre <= 12, "slices must follow the MFMAs that read their P");
#pragma unroll
    for (int i = 0; i < kNv; ++i) {
      const int u = i / G::kNcb;
      oacc[i % G::kNcb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          vf[i % kPf], __builtin_bit_cast(bf16x8, pb[u >> 1][u & 1]), oacc[i % G::kNcb], 0, 0, 0);
      if (i + kPf < kNv) vf[i % kPf] = vfrag(vb, i + kPf);
      if constexpr (decltype(with_next)::value && kPre > 0) {
        // the exponentials make this part vector-heavy like phase A: priority
        // 1 again (measured +0.3-0.7% on the headline)
        if (i == kB0) __builtin_amdgcn_s_setprio(1);
        if (i >= kB0) {
#pragma unroll
          for (int k = kPer * (i - kB0); k < kPer * (i + 1 - kB0); ++k)
            exp_slice(sn, pb, m_use, rs_next, k);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto qk_plain = [&](const uint8_t* kb, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 kf[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) kf[i] = kfrag(kb, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kNq; ++i) {
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % kPf], qf[i >> 1], s[i & 1], 0, 0, 0);
      if (i + kPf < kNq) kf[i % kPf] = kfrag(kb, i + kPf);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // P of the current tile (bf16 pairs): pb[0] = keys 0..31, written by the
  // previous iteration's phase B (or the prologue), pb[1] = keys 32..63,
  // written by phase A; rs_half: the first half's probability sum.
  u32x4 pb[2][2];
  float rs_half = 0.f;
  // has_next (compile time): tile j+1 exists. The last tile gets its own
  // code so the compiler cannot merge its exponentials with the pipelined
  // ones and pull them out of the MFMA slots.
  auto iteration = [&](auto has_next, int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    constexpr bool kNext = decltype(has_next)::value;
    const int cur = j & 1;
    // K_{j+2} and V_{j+1} go straight into the buffers of K_j and V_{j-1},
    // one DMA instruction beside every (kNq / kNdma)-th S^T MFMA so that the
    // eight waves do not all queue their loads at once. Past the last tile
    // the last K tile is fetched again into the free buffer (branch-free;
    // nobody reads it).
    const uint8_t* kt = nullptr;
    const uint8_t* vt = nullptr;
    if constexpr (kNext) {
      kt = prep_k(min(j + 2, nt - 1));
      vt = prep_v(j + 1);
    }
    uint8_t* const kd = kbuf + cur * G::kKBytes;
    uint8_t* const vd = vbuf + (cur ^ 1) * G::kVBytes;
    auto dma = [&](int slot) {
      if constexpr (kNext) {
#pragma unroll
        for (int n = 0; n < kNdma; ++n) {
          if ((n * kNq) / kNdma != slot) continue;
          if (n < G::kDmaPerWave) dma_k(kt, kd, n);
          else dma_v(vt, vd, n - G::kDmaPerWave);
        }
      }
    };
    // a row with no reference yet exponentiates against 0 and takes the
    // rare path below
    // Causal or window edge: the O^T product of a tile whose every key lies
    // outside the visible range of all 32 rows of this wave is skipped (its
    // scores are all masked to -inf, so its probabilities are exactly 0 and
    // the product would add nothing); the workgroup still copies the tile
    // for its other waves.
    static_assert(!CAUSAL || kPre == 0, "a skipped phase B would drop the next tile's slices");
    auto seen = [&](int t) {
      const int kv0 = ktile(t) * kBc;
      return kv0 <= qmax_w + off && (!LOCAL || kv0 + kBc - 1 >= qmin_w + off_l);
    };
    float rs = rs_half + phase_a(has_next, klane + (cur ^ 1) * G::kKBytes, sc, sn, pb,
                                 m_run == -INFINITY ? 0.f : m_run, dma);
    if (__builtin_amdgcn_ballot_w64(!(rs <= kBig) || m_run == -INFINITY) != 0) {
      // rare: move the reference to the tile maximum (never down) and redo
      // the tile; alpha = 0 for a row that had no reference (O, l are 0)
      const float r_new = fmaxf(m_run, tile_max(sc));
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - r_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      m_run = r_new;
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      rs = 0.f;
#pragma unroll
      for (int k = 0; k < kSlices; ++k) exp_slice(sc, pb, m_use, rs, k);
    }
    l_run += rs;
    rs_half = 0.f;
    if constexpr (kNext) mask_bias(j + 1, sn);
    if (!CAUSAL || seen(j))
      phase_b(has_next, vlane + cur * G::kVBytes, pb, sn, m_run == -INFINITY ? 0.f : m_run, rs_half);
    if constexpr (kNext) {
      // a bias block copied above (tile j+2 exists) may stay in flight
      if (bias_dma && j + 2 < nt)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        wait_tiles();
      __syncthreads();
    }
  };
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;

  f32x16 sa[2], sb[2];
  if (nt > 0) {
    // K_0 and the first bias block, then V_0 and K_1: the first two are
    // waited for (copies complete in issue order) and the last two may land
    // while S_0 is computed
    load_k(0);
    if (bias_dma) dma_bias(0);
    load_v(0);
    if (nt > 1) {
      load_k(1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G::kDmaPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(G::kDmaPerWave) : "memory");
    }
    __syncthreads();
    qk_plain(klane, sa);
    // iteration 0 reads V_0 (and K_1) and overwrites K buffer 0 (with K_2,
    // or with K_1 again when there are two tiles): every wave's copies have
    // landed and every wave is done reading K_0
    wait_tiles();
    __syncthreads();
    mask_bias(0, sa);
    m_run = tile_max(sa);
    // the slices of tile 0 computed ahead (the later tiles' come from the
    // phase B before them)
    {
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int k = 0; k < kPre; ++k) exp_slice(sa, pb, m_use, rs_half, k);
    }
    int j = 0;
    for (; j + 2 < nt; j += 2) {
      iteration(Yes{}, j, sa, sb);
      iteration(Yes{}, j + 1, sb, sa);
    }
    if (nt - j == 2) {
      iteration(Yes{}, j, sa, sb);
      iteration(No{}, j + 1, sb, sa);
    } else {
      iteration(No{}, j, sa, sb);
    }
  }

  // ---- epilogue: one division per row, O and LSE written once
  const float l_tot = lane_pair_sum(l_run);
  if constexpr (SPLIT) {
    if (!row_live) return;
    // one split of the keys: its normalised output and log-sum-exp in fp32,
    // merged with the other splits by the combine kernel
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int64_t row = (((int64_t)split * p.B + b) * p.H + row_h) * Nq + row_i;
    float* orow = p.part_o + row * D;
#pragma unroll
    for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[cb][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g + 4 * hi) = w;
      }
    if (hi == 0)
      p.part_lse[row] = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  } else if (my_q < Nq) {  // not split: the final result
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    __bf16* orow = static_cast<__bf16*>(p.o) + (VARLEN ? q_lo * p.o_sn : b * p.o_sb) + h * p.o_sh +
                   (int64_t)my_q * p.o_sn;
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
      float* lrow = p.lse + (VARLEN ? q_lo : b * p.l_sb) + h * p.l_sh;
      lrow[my_q] = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
  }  // items
}

template <int D, int W, bool CAUSAL, bool HAS_BIAS, bool SPLIT, bool LOCAL, bool VARLEN>
hipError_t launch_one(const FwdParams& p, const TileMap& tm, hipStream_t stream) {
  using G = Geo<D, W>;
  // d = 64 biased kernels also hold the staged bias blocks
  constexpr int kSmemAll = G::kSmem + ((HAS_BIAS && D == 64) ? G::kBiasBytes : 0);
  static bool attr_set = false;  // benign race: every caller sets the same value
  auto kern = fwd_bf16_kernel<D, W, CAUSAL, HAS_BIAS, SPLIT, LOCAL, VARLEN>;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmemAll);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = 8 * tm.per_xcd;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(G::kThreads), kSmemAll, stream, p, tm);
  return hipGetLastError();
}

// Dispatch over head dimension, workgroup size, mask kind and bias for one
// family of instantiations (each family is compiled in its own source file).
template <bool SPLIT, bool LOCAL, bool VARLEN = false>
hipError_t launch_family(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  auto go = [&](auto dc, auto wc) -> hipError_t {
    constexpr int D = decltype(dc)::value, W = decltype(wc)::value;
    if constexpr (VARLEN) {
      if (p.bias != nullptr) return hipErrorInvalidValue;
      if (LOCAL || p.causal) return launch_one<D, W, true, false, false, LOCAL, true>(p, tm, s);
      if constexpr (!LOCAL) return launch_one<D, W, false, false, false, false, true>(p, tm, s);
      return hipErrorInvalidValue;
    } else {
      const bool bias = p.bias != nullptr;
      if (LOCAL || p.causal)
        return bias ? launch_one<D, W, true, true, SPLIT, LOCAL, false>(p, tm, s)
                    : launch_one<D, W, true, false, SPLIT, LOCAL, false>(p, tm, s);
      if constexpr (!LOCAL)
        return bias ? launch_one<D, W, false, true, SPLIT, false, false>(p, tm, s)
                    : launch_one<D, W, false, false, SPLIT, false, false>(p, tm, s);
      return hipErrorInvalidValue;
    }
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  using W4 = std::integral_constant<int, 4>;
  using W8 = std::integral_constant<int, 8>;
  if (d == 128) {
    // 4-wave workgroups for d = 128 are only chosen for split launches
    if constexpr (SPLIT)
      if (waves == 4) return go(D128{}, W4{});
    return go(D128{}, W8{});
  }
  if (d == 64) return waves == 4 ? go(D64{}, W4{}) : go(D64{}, W8{});
  return hipErrorInvalidValue;
}

}  // namespace

// One function per family, each defined in its own source file.
hipError_t launch_bf16_plain(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s);
hipError_t launch_bf16_split(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s);
hipError_t launch_bf16_local(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s);
hipError_t launch_bf16_varlen(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s);
// Persistent form for dense, causal and window problems
// (fwd_bf16_stream.hip): `grid` workgroups, one per compute unit, each
// walking several query tiles as one stream of key tiles of `key_tile` keys
// (64, or 128 for dense problems at d = 64).
hipError_t launch_bf16_stream(const FwdParams& p, const TileMap& tm, int d, int key_tile, int grid,
                              hipStream_t s);

}  // namespace attn
