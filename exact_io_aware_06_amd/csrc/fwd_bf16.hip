// bf16 forward: the unsplit, unwindowed instantiations and the host-side
// dispatch of every bf16 launch (tile map, workgroup size, family). The
// kernel itself is in fwd_bf16_kernel.h; the split and window families are
// compiled in fwd_bf16_split.hip, fwd_bf16_local.hip and
// fwd_bf16_local_split.hip.

#include "fwd_bf16_kernel.h"

namespace attn {

hipError_t launch_bf16_plain(const FwdParams& p, const TileMap& tm, int d, int waves, hipStream_t s) {
  return launch_family<false, false>(p, tm, d, waves, s);
}

int fwd_bf16_pack(int64_t head_group, int64_t nq) {
  // decoding-sized query counts only: with many rows per head the packed
  // row space would also blur the causal tile skipping
  return (head_group > 1 && nq <= 64) ? (int)head_group : 1;
}

int fwd_bf16_rows(int d, int64_t nrows, bool causal, bool bias, bool split) {
  // d = 64 with a causal mask or a bias: 4-wave (128-row) workgroups, so
  // that two run on a CU at once and the uneven per-workgroup work (diagonal
  // tiles, per-batch key lengths) is spread more finely. A split launch with
  // at most 128 query rows (decoding) also takes 4 waves: the rows past Nq
  // are wasted matrix work, and 4-wave workgroups put half as much of it on
  // each SIMD. Otherwise 8 waves.
  if (d == 64 && (causal || bias)) return 128;
  if (split && nrows <= 128) return 128;
  return 256;
}

// Compute units of the current device (cached per device; 256 on MI355X).
static int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Packed sequences take the persistent form (64-key tiles) with no window,
// at most 64 sequences, H a multiple of 8 (H/8 heads of every sequence per
// XCD), at most 2048 query tiles per head (B * ceil(max_q / 256)), at least
// 64 keys in all (a sequence's last key tile is read shifted inside the
// packed keys) and rows in reach of 32-bit copy offsets.
static int stream_grid_varlen(const FwdParams& p, int kt) {
  if (kt != 64 || p.local || p.bias != nullptr || p.kv_len != nullptr || p.n_split > 1) return 0;
  if (p.B < 1 || p.B > 64 || p.H < 8 || p.H % 8 != 0 || p.Nk < 64 || p.max_q < 1) return 0;
  if ((int64_t)p.B * ((p.max_q + 255) / 256) > 2048) return 0;
  for (int64_t sn : {p.q_sn, p.k_sn, p.v_sn})
    if (64 * sn * 2 >= ((int64_t)1 << 31)) return 0;
  const int cus = device_cus();
  return cus % 8 == 0 ? cus : 0;
}

// Padded batches with a bias take the persistent form's work list with batch
// b as sequence b (64-key tiles, keys kv_len[b] or Nk) at d = 64 without a
// causal mask or window, when the bias blocks can be copied by LDS DMA
// (bias_dma: rows 16-byte aligned, Nk a multiple of 4), at most 64 batches,
// H a multiple of 8, at least 64 keys, at most 2048 query tiles per head
// (B * ceil(Nq / 256)), rows in reach of 32-bit copy offsets and at least
// two query tiles per compute unit.
static int stream_grid_bias(const FwdParams& p, int d, int kt) {
  if (d != 64 || kt != 64 || p.causal || p.local || p.n_split > 1 || !p.bias_dma) return 0;
  if (p.B < 1 || p.B > 64 || p.H < 8 || p.H % 8 != 0 || p.Nk < 64) return 0;
  const int64_t nqt = (p.Nq + 255) / 256;
  if ((int64_t)p.B * nqt > 2048) return 0;
  for (int64_t sn : {p.q_sn, p.k_sn, p.v_sn})
    if (64 * sn * 2 >= ((int64_t)1 << 31)) return 0;
  const int cus = device_cus();
  if (cus % 8 != 0 || (int64_t)p.B * p.H * nqt < 2 * (int64_t)cus) return 0;
  return cus;
}

// The persistent form (fwd_bf16_stream.hip), 256-row query tiles and one
// workgroup per compute unit, streams key tiles of kt keys (64, or 128 at
// d = 64). Unpacked and unbiased, it applies with no key lengths or key split,
// when every key tile is full and they come in pairs (Nk a
// multiple of 2 kt), rows are in reach of 32-bit copy offsets and there are
// at least two query tiles per compute unit. Dense query tiles host the next
// one's Q copy during their first key tiles and need at least 14 of them at
// d = 128 (8 at d = 64). Causal problems also need the diagonal on key-tile
// pairs (Nk >= Nq, Nk - Nq a multiple of 2 kt) and B*H a multiple of 8
// (whole heads per XCD); windows need Nk >= Nq; short causal and window
// tiles copy at once. Returns the grid, or 0.
static int stream_grid(const FwdParams& p, int d, int kt) {
  if (p.cu_q != nullptr) return stream_grid_varlen(p, kt);
  if (p.bias != nullptr) return stream_grid_bias(p, d, kt);
  if (p.n_split > 1 || p.kv_len != nullptr) return 0;
  if (p.Nk % (2 * kt) != 0 || 64 * p.q_sn * 2 >= ((int64_t)1 << 31)) return 0;
  const int cus = device_cus();
  if (cus % 8 != 0) return 0;
  const int64_t n_qtiles = (p.Nq + 255) / 256;
  const int64_t total = (int64_t)p.B * p.H * n_qtiles;
  if (total < 2 * (int64_t)cus) return 0;
  if (!p.causal) return p.Nk / kt >= (d == 128 ? 14 : 8) ? cus : 0;
  const int64_t off = p.Nk - p.Nq;
  if (p.local) return off >= 0 ? cus : 0;
  if (off < 0 || off % (2 * kt) != 0 || ((int64_t)p.B * p.H) % 8 != 0) return 0;
  return cus;
}

// Key tile of the persistent form: 128 keys for dense problems at d = 64
// (half the per-tile checks, waits and barriers per key; the K/V buffers
// take the 64 KiB of a d = 128 tile; measured 1.2-1.3% faster at
// N = 2048 and 4096), else 64 (with a causal diagonal or a window edge, a
// 128-key tile masks twice as much work: 2-3% slower).
static int stream_key_tile(const FwdParams& p, int d) {
  return (d == 64 && !p.causal && stream_grid(p, d, 128) > 0) ? 128 : 64;
}

int launch_fwd_bf16(const FwdParams& p_in, int d, void* stream) {
  FwdParams p = p_in;
  const bool split = p.n_split > 1;
  const bool packed = split && p.pack > 1;
  const bool varlen = p.cu_q != nullptr;
  // rows of one row space: Nq, pack * Nq, or the longest packed sequence
  const int64_t nrows = varlen ? p.max_q : packed ? (int64_t)p.pack * p.Nq : p.Nq;
  const int br = fwd_bf16_rows(d, nrows, p.causal != 0, p.bias != nullptr, split);
  const int waves = br / 32;
  TileMap tm{};
  tm.n_qtiles = (int)((nrows + br - 1) / br);
  const int64_t total = (int64_t)p.B * (packed ? p.Hk : p.H) * tm.n_qtiles;
  tm.total = (int)total;
  tm.per_xcd = (int)((total + 7) / 8);
  tm.batch_inner = (p.bias != nullptr && p.bias_sb == 0 && p.B > 1) ? 1 : 0;
  tm.reverse_q = p.causal ? 1 : 0;
  tm.n_split = 1;
  // causal tiles differ in length: deal heads in groups, longest tiles
  // first (8 / waves workgroups fit on a CU: two waves per SIMD)
  tm.group = p.causal ? dispatch_group(tm.n_qtiles, 8 / waves) : 1;
  if (p.n_split > 1) {
    tm.n_split = p.n_split;
    const int64_t all = total * p.n_split;
    tm.total = (int)all;
    tm.per_xcd = (int)((all + 7) / 8);
    tm.batch_inner = 0;
  }
  // Paired batches for d = 64 with a batch-broadcast bias and key lengths
  // (the kernel ranks the batches by key length on the device; B <= 64 so
  // that one wavefront holds them)
  if (d == 64 && !split && !varlen && !p.causal && !p.local && p.bias != nullptr &&
      p.bias_sb == 0 && p.kv_len != nullptr && p.B >= 2 && p.B <= 64) {
    tm.pairs = (p.B + 1) / 2;
    const int64_t all = (int64_t)p.H * tm.n_qtiles * tm.pairs;
    tm.total = (int)all;
    tm.per_xcd = (int)((all + 7) / 8);
    tm.batch_inner = 0;
  }
  if (varlen) {
    // groups of query tiles dealt round-robin over the XCDs (decode_tile),
    // longest sequences first when they can be ranked in one wavefront
    const int64_t groups = (int64_t)p.B * p.H;
    tm.per_xcd = (int)((groups + 7) / 8 * tm.n_qtiles);
    tm.rank_seq = p.B <= 64 ? 1 : 0;
  }
  // d = 64 biased kernels stage each wave's 32 bias rows in LDS by DMA when
  // every row start is 16-byte aligned, whole 4-key chunks cover the keys,
  // rows belong to one head (no packing) and 32 rows fit 32-bit offsets
  p.bias_dma = (p.bias != nullptr && d == 64 && p.bias_vec && p.Nk >= 4 && p.Nk % 4 == 0 &&
                !packed && 32 * p.bias_sn * 4 + 256 < ((int64_t)1 << 31)) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (const int kt = stream_key_tile(p, d), grid = stream_grid(p, d, kt); grid > 0) {
    TileMap ts{};
    ts.n_qtiles = (int)(((varlen ? p.max_q : p.Nq) + 255) / 256);
    ts.total = (int)((int64_t)p.B * p.H * ts.n_qtiles);
    ts.per_xcd = (ts.total + 7) / 8;
    return (int)launch_bf16_stream(p, ts, d, kt, grid, s);
  }
  if (varlen) return (int)launch_bf16_varlen(p, tm, d, waves, s);
  if (p.local) return (int)launch_bf16_local(p, tm, d, waves, s);
  return split ? (int)launch_bf16_split(p, tm, d, waves, s) : (int)launch_bf16_plain(p, tm, d, waves, s);
}

}  // namespace attn
