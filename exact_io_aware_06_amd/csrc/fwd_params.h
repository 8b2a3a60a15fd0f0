// Internal parameter block handed from the C ABI front end to the kernel
// launchers. Plain data: every pointer is a device pointer, strides are in
// elements and already validated (non-negative, alignment checked).
#pragma once

#include <stdint.h>

#include "attn.h"

namespace attn {

// Size of the per-device scratch array behind attn_fwd_splitkv_noalloc.
constexpr int64_t kNoallocScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
// The calling thread's current device's address of that array (fetched with
// hipGetSymbolAddress on the first call on the device). Returns a hipError_t.
int noalloc_scratch(void** ptr);

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* bias;      // nullptr when absent
  const int32_t* kv_len;  // nullptr when absent

  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t l_sb, l_sh;        // lse: row stride is 1
  int64_t bias_sb, bias_sh, bias_sn;  // 0 for a broadcast dimension

  int32_t B, H, Hk, Nq, Nk;
  int32_t head_group;        // H / Hk
  int32_t causal;
  int32_t bias_vec;          // 1: every bias row start is 16-byte aligned
  int32_t bias_dma;          // 1: d = 64 kernels stage bias tiles in LDS (set
                             // by the launcher: bias_vec, Nk % 4 == 0, no
                             // packed heads, 32 rows and a row within 2 GiB)
  float scale_log2;          // scale * log2(e): scores go to base-2 units
  float scale;               // the softmax scale itself (biased kernels)

  // Split over keys (flash-decoding). n_split == 1: each workgroup covers all
  // keys of its query tile and writes o / lse. n_split > 1: a workgroup
  // covers keys [s * kv_split, (s + 1) * kv_split) of one split s and writes
  // its normalised partial output and log-sum-exp (natural log) to
  // part_o[s][b][h][i][:] and part_lse[s][b][h][i] (fp32, contiguous);
  // the combine kernel then merges the splits into o / lse.
  int32_t kv_split;          // keys per split, a multiple of 64
  int32_t n_split;
  float* part_o;             // [n_split, B, H, Nq, d]
  float* part_lse;           // [n_split, B, H, Nq]
  // Split launches only: > 1 packs the `pack` (= H / Hk) query heads that
  // share a key/value head into one row space of pack * Nq rows per
  // (batch, key/value head), so each workgroup reads K/V once for all of
  // them. 1: one row space of Nq rows per query head.
  int32_t pack;
  // Sliding window (local attention): local != 0 hides key j from query i
  // unless i + (Nk - Nq) - win_left <= j <= i + (Nk - Nq) + win_right. Both
  // bounds are >= 0 (an open side is given as a bound that excludes
  // nothing). Launched on the causal instantiations (causal is a window
  // with win_right = 0 and no left bound).
  int32_t local;
  int32_t win_left;
  int32_t win_right;
  // Packed variable-length sequences: non-null cu_q / cu_k (device, int32
  // [B + 1]) give sequence b the rows [cu_q[b], cu_q[b+1]) of the packed
  // query rows (Nq of them in all) and the keys [cu_k[b], cu_k[b+1]) of the
  // packed keys (Nk in all); B counts sequences, the batch strides are 0 and
  // the grid covers max_q rows per sequence.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t max_q;
};

// Parameter block of the backward (bf16). Same conventions as FwdParams;
// q, o, do_, dq are [B, H, Nq, d], k, v, dk, dv are [B, Hk, Nk, d]; lse is
// the forward's natural log-sum-exp [B, H, Nq]. The workspace holds, per
// query row, D = rowsum(dO o O) and the log-sum-exp in base 2 (+inf for a
// row with no visible key, so that every probability it recomputes is 0).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* do_;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  const float* bias;
  const int32_t* kv_len;
  float* dsum;   // [B, H, Nq]: D
  float* lse2;   // [B, H, Nq]: -lse * log2(e) (-inf for a row that saw no key)

  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int64_t l_sb, l_sh;
  int64_t bias_sb, bias_sh, bias_sn;

  int32_t B, H, Hk, Nq, Nk;
  int32_t head_group;
  int32_t causal;      // right-bounded mask (also set for a window)
  int32_t local;       // window: left bound as well
  int32_t win_left, win_right;
  float scale;
  float scale_log2;
};

int launch_bwd_bf16(const BwdParams& p, int d, void* stream);
// Zero fill of a strided bf16 [B, H, N, d] tensor (rows 16-byte aligned).
int launch_zero_bf16(void* data, int64_t B, int64_t H, int64_t N, int d, int64_t sb,
                     int64_t sh, int64_t sn, void* stream);

// How the flat workgroup index maps onto (batch, head, query tile).
struct TileMap {
  int32_t n_qtiles;      // ceil(Nq / tile rows)
  int32_t total;         // B * H * n_qtiles
  int32_t per_xcd;       // ceil(total / 8)
  int32_t batch_inner;   // 1: batch index varies fastest (shared bias reuse)
  int32_t reverse_q;     // 1: longest query tiles first (causal)
  int32_t n_split;       // key splits per query tile (1: no split)
  int32_t group;         // > 1: flat (batch, head) indices dealt in groups of
                         // this many, tile index slow within a group
  int32_t pairs;         // > 0: paired batches (d = 64, broadcast bias, key
                         // lengths): pairs per (head, query tile), the
                         // workgroup of pair r runs the batches of key-length
                         // rank r and B-1-r; total = H * n_qtiles * pairs
  int32_t rank_seq;      // 1: packed sequences (B <= 64) dealt in decreasing
                         // order of query x key length
};

// Number of flat heads to deal together so that one XCD's resident
// workgroups (32 CUs x wg_per_cu) cover the longest tiles of a whole group
// before any shorter one: ceil(32 wg_per_cu / n_tiles), at least 1.
inline int32_t dispatch_group(int n_tiles, int wg_per_cu) {
  if (n_tiles <= 0) return 1;
  const int slots = 32 * wg_per_cu;
  return slots > n_tiles ? (slots + n_tiles - 1) / n_tiles : 1;
}

// Host-side launchers (one per kernel family). Return a hipError_t value.
int launch_fwd_bf16(const FwdParams& p, int d, void* stream);
int launch_fwd_f32(const FwdParams& p, int d, void* stream);
// Merge of the n_split partial results of a split launch into o / lse (bf16 o).
int launch_combine_bf16(const FwdParams& p, int d, void* stream);
// Query rows per workgroup of the bf16 forward. nrows: rows of one row
// space (Nq, or pack * Nq when heads are packed); split: a split-key launch.
int fwd_bf16_rows(int d, int64_t nrows, bool causal, bool bias, bool split);
// Heads packed per row space for a split launch (1: none).
int fwd_bf16_pack(int64_t head_group, int64_t nq);

}  // namespace attn
