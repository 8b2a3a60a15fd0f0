// bf16 forward, persistent ("stream") form for problems with no bias, key
// lengths or key split, every key tile full (Nk a multiple of 128): dense,
// causal with the diagonal on key-tile pairs, or a sliding window; for
// packed variable-length sequences (dense or causal, per sequence); and for
// padded batches with an additive bias and key lengths at d = 64.
//
// Same arithmetic as fwd_bf16_kernel.h (transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, base-2 exponentials against an overflow-checked
// reference, O^T += V^T P^T from LDS transpose reads; "Understanding
// FlashAttention Pt 1", sections 2.3-2.4 and 3.1), with the query tiles of
// a workgroup processed back to back as one stream of key tiles.
//
// Why: with one workgroup per query tile, every round of workgroups starts
// with all compute units loading their Q rows and first key/value tiles at
// once and ends with all of them writing O at once; measured on the
// B=2 H=32 N=4096 d=128 workload, those two bursts took about 11k and 7k of
// a workgroup's 209k cycles, in every round. Here one workgroup per compute
// unit walks its query tiles in turn (the tiles of one XCD stay on it, as in
// the per-tile launch) and the boundary between two tiles costs about one
// ordinary iteration:
//   * the next tile's Q rows are copied into LDS by LDS DMA, one 1 KB copy
//     per wavefront per iteration, early in the current tile;
//   * the key/value stream runs across the boundary: the last iteration of
//     a tile already copies the next tile's first key/value tiles and
//     computes the next tile's first S^T (with the next Q, read from LDS);
//   * the finished tile's O is normalised and written to LDS (each
//     wavefront into its own 32 rows, where its Q rows were), then copied
//     out in whole 16-byte row pieces during the next tile's first
//     iterations, two copies per wavefront per iteration, so full 256-byte
//     rows leave each instruction and the writes are spread over time.
// Rows of Q/O in LDS: row r at r * 2d bytes, 16-byte chunk c at slot
// c ^ (r mod d/8), so that the 16 lanes of a transposing read or of a row
// copy hit 16 different bank groups.
//
// Key tiles hold 64 keys (NB = 2 blocks of 32), or 128 (NB = 4) for dense
// problems at d = 64, whose vector work per MFMA is twice that of d = 128:
// the per-tile overflow check, copy waits and barrier then come half as
// often per key.
//
// Causal (bottom-right aligned: key j hidden from query i when
// j > i + Nk - Nq; "Understanding FlashAttention Pt 1", section 3.5): query
// tile t sees the key tiles up to its diagonal, 4 (t + 1) + (Nk - Nq) / 64
// of them, so the tiles differ in length and a workgroup's share has to be
// balanced ahead of time. Each XCD takes B*H/8 whole heads; their query
// tiles, longest first, are dealt to the XCD's workgroups in rounds, the
// direction alternating from round to round, so that every workgroup's
// total is about the same and its own tiles come longest first. A tile
// too short to spread the previous O's drain and the next Q's copy over its
// iterations does both at its start.
// The score tiles that cross a wavefront's diagonal are masked to -inf
// before their exponentials; every row sees key 0, so no row is empty.
//
// Window (key j kept for query i iff i + Nk - Nq - left <= j <= i + Nk - Nq
// + right; Nk >= Nq): the tiles are dealt as for dense problems, each
// covering the key tiles from the left edge of its first row to the right
// edge of its last (made even by one more masked tile), visited in a
// rotated order: step t reads the tile whose absolute index is congruent
// to t modulo their number, so neighbouring query tiles of a head, running
// side by side on an XCD, read each key tile at the same step. Scores
// outside either edge are masked; every row sees key i + Nk - Nq. A row's
// first visited tile can be hidden from it: its reference stays unset
// (-inf) and the overflow check's rare path sets it at the first tile it
// sees.

//
// Packed sequences ("flash-attention", Part II, variable-length batches):
// the work list of (sequence, head, query tile) is built in LDS by every
// workgroup at its start (longest tiles first, ranked in closed form), XCD
// x takes heads x H/8 .. (x + 1) H/8 - 1 of every sequence, and its
// workgroups deal the list greedily by the work they already hold. Key
// tiles are a sequence's own keys in 64-key steps; the last one, read
// shifted to end inside the packed keys, is masked to the keys it owns.
//
// Padded batches with a bias (d = 64, not causal; BIAS): the same work list
// with batch b as sequence b (all Nq query rows, key count kv_len[b] or Nk)
// and the batch strides of the tensors; key tiles are read in place (the
// last 64 keys of the tensor for a tile reaching past them). Each wavefront
// copies the fp32 bias block of its 32 rows for the next key tile into its
// own 8 KB of LDS by DMA (no other wavefront reads it) right after reading
// the current one, which it adds to the raw scores as scale * qk + bias
// (natural units, one FMA; the exponentials then take log2(e)). The copy is
// the iteration's last vector memory operation and may stay in flight
// across the barrier: it is waited for where the next block is read.

#include "fwd_bf16_kernel.h"

namespace attn {
namespace {

// NB: 32-key blocks per key tile (2: 64 keys, 4: 128 keys).
// Packed sequences (VARLEN): at most kMaxSeqs sequences and kMaxEntries
// query tiles of one head in all, listed in LDS behind the K/V and Q/O rows.
constexpr int kMaxSeqs = 64;
constexpr int kMaxEntries = 2048;
constexpr int kGreedyRounds = 16;                 // greedy deal up to this many items per workgroup
constexpr int kGreedyItems = kGreedyRounds * 64;  // (at most 64 workgroups per XCD)
constexpr int kSeqTableBytes =
    24 * kMaxSeqs + 4 * kMaxEntries + 4 * kGreedyItems + 4 * 64 + 4 * (kGreedyRounds + 1) + 16;

// LDS of the bias blocks (BIAS): one 8 KB block of 32 rows x 64 keys (fp32)
// per wavefront, behind the K/V buffers, Q/O rows and the work list.
constexpr int kBiasWave = 32 * 64 * 4;
template <int D, int NB>
constexpr int bias_lds_offset() {
  return (4 * (32 * NB) * D * 2 + 8 * 32 * 2 * D + kSeqTableBytes + 255) / 256 * 256;
}

template <int D, int NB, bool CAUSAL, bool LOCAL, bool VARLEN, bool BIAS>
__global__ __launch_bounds__(512, 2) void fwd_bf16_stream_kernel(FwdParams p, TileMap tm) {
  static_assert(CAUSAL || !LOCAL, "a window is a two-sided causal mask");
  static_assert(NB == 2 || NB == 4, "64- or 128-key tiles");
  static_assert(!VARLEN || (NB == 2 && !LOCAL), "packed sequences: 64-key tiles, no window");
  static_assert(!BIAS || (VARLEN && D == 64 && !CAUSAL), "bias: padded batches at d = 64, not causal");
  constexpr int W = 8;
  using G = Geo<D, W>;
  constexpr int kKT = 32 * NB;                  // keys per key tile
  constexpr int kKBytes = kKT * D * 2;          // one K (or V) tile in LDS
  constexpr int kSmemKV = 4 * kKBytes;          // two K and two V buffers
  constexpr int kDmaPerWave = kKBytes / 1024 / W;  // 1 KB copies per wave per tile
  constexpr int kBr = G::kBr;                   // 256 query rows per tile
  constexpr int kC = D / 8;                     // 16-byte chunks per row
  constexpr int kRowBytes = 2 * D;
  constexpr int kQWave = 32 * kRowBytes;        // a wavefront's Q / O rows in LDS
  constexpr int kQCopies = kQWave / 1024;       // 1 KB copies for them (D / 16)
  constexpr int kRowsPerKB = 1024 / kRowBytes;  // rows per 1 KB (4 or 8)
  constexpr int kDrainIters = (kQCopies + 1) / 2;  // O copied out, 2 per iteration
  constexpr int kQ0 = kDrainIters;              // first iteration copying the next Q
  constexpr int kSmemRows = kSmemKV + W * kQWave;  // K/V buffers and Q/O rows
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Tiles of this workgroup (workgroup w runs on XCD w % 8). Dense and
  // window: the logical tiles slot, slot + wpx, ... of its XCD's range.
  // Causal: round r gives it the tile at position slot (r even) or
  // wpx - 1 - slot (r odd) of the r-th group of wpx in its XCD's tiles
  // sorted longest first.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, wpx = gridDim.x >> 3;
  const int base_logical = xcd * tm.per_xcd + slot;
  // heads per XCD: causal, of the B*H (batch, head) pairs; packed sequences,
  // of the H heads (XCD x takes heads x H/8 .. (x + 1) H/8 - 1 of every
  // sequence, so every XCD gets the same work)
  const int hpx = VARLEN ? (p.H >> 3) : ((p.B * p.H) >> 3);

  // Packed sequences: every workgroup lists the query tiles (b, t) of one
  // head, t < min(ceil(rows_b / 256), tm.n_qtiles), longest first, in LDS:
  // seq[b] = (rows, keys, tiles) and sbase[b] = (first row, first key) of
  // sequence b, ent[r] = t * 64 + b for the tile of rank r, icost[i] the
  // work of item i of the XCD's (tile, head) list in half key tiles. A
  // tile's length is the number of 64-key tiles its rows see; it is
  // non-decreasing in t within a sequence, so the number of tiles of
  // sequence b' longer than v has a closed form (cnt_gt), and a tile's rank (by
  // length descending, then sequence ascending, then t descending) is a sum
  // of such counts over the sequences.
  int4* const seq = reinterpret_cast<int4*>(smem + kSmemRows);
  int2* const sbase = reinterpret_cast<int2*>(smem + kSmemRows + 16 * kMaxSeqs);
  int* const ent = reinterpret_cast<int*>(smem + kSmemRows + 24 * kMaxSeqs);
  int* const icost = ent + kMaxEntries;
  int* const gkey = icost + kGreedyItems;   // greedy deal: the workgroups' keys (16-byte aligned)
  int* const mine = gkey + 64;              // greedy deal: this workgroup's items, then their count
  int* const nent = mine + kGreedyRounds + 1;
  int n_ent = 0;
  if constexpr (VARLEN) {
    const int nqt = tm.n_qtiles;
    if (tid < 64) {
      // one wavefront (B <= 64): the sequences, and their tiles in all
      int nq = 0;
      if (tid < p.B) {
        int a0 = 0, c0 = 0, lq = p.Nq, lk = p.Nk;
        if constexpr (BIAS) {
          // batch tid: every query row, kv_len[tid] keys (clamped) or all
          if (p.kv_len != nullptr) lk = min(max(p.kv_len[tid], 0), p.Nk);
        } else {
          a0 = min(max(p.cu_q[tid], 0), p.Nq);
          const int a1 = min(max(p.cu_q[tid + 1], a0), p.Nq);
          c0 = min(max(p.cu_k[tid], 0), p.Nk);
          const int c1 = min(max(p.cu_k[tid + 1], c0), p.Nk);
          lq = a1 - a0;
          lk = c1 - c0;
        }
        nq = min((lq >> 8) + ((lq & 255) != 0 ? 1 : 0), nqt);
        seq[tid] = make_int4(lq, lk, nq, 0);
        sbase[tid] = make_int2(a0, c0);
      }
      int tot = nq;
#pragma unroll
      for (int dd = 32; dd >= 1; dd >>= 1) tot += __shfl_xor(tot, dd, 64);
      if (tid == 0) nent[0] = tot;
    }
    __syncthreads();
    n_ent = __builtin_amdgcn_readfirstlane(nent[0]);
    // 64-key tiles seen by the rows of tile t (all keys without a mask)
    auto length = [&](int lq, int lk, int t) {
      int kv = lk;
      if (CAUSAL) kv = min(lk, min(kBr * (t + 1), lq) + (lk - lq));
      return (max(kv, 0) + kKT - 1) / kKT;
    };
    // tiles of a sequence longer than v (v >= -1)
    auto cnt_gt = [&](const int4& sq, int v) {
      if (v < 0) return sq.z;
      if (sq.y <= kKT * v) return 0;
      if (!CAUSAL) return sq.z;
      return max(0, sq.z - max(0, (kKT * v - (sq.y - sq.x)) >> 8));
    };
    for (int e = tid; e < p.B * nqt; e += 512) {
      const int b = e / nqt, t = e - b * nqt;
      const int4 sb = seq[b];
      if (t >= sb.z) continue;
      const int v = length(sb.x, sb.y, t);
      int rank = sb.z - 1 - t - cnt_gt(sb, v);
#pragma unroll 8
      for (int b2 = 0; b2 < p.B; ++b2) {
        const int4 s2 = seq[b2];
        const int g = cnt_gt(s2, v);
        rank += g + (b2 < b ? cnt_gt(s2, v - 1) - g : 0);
      }
      ent[rank] = (t << 6) | b;
      // its work: the key tiles it runs (even, at least 2) plus about 2.5
      // tiles of start and diagonal (measured), in half tiles
      const int cost = 2 * max(2, v + (v & 1)) + 5;
      for (int h = 0; h < hpx; ++h)
        if (rank * hpx + h < kGreedyItems) icost[rank * hpx + h] = cost;
    }
    __syncthreads();
  }

  int n_items;
  // packed sequences with at most kGreedyRounds items per workgroup: a
  // greedy deal (below), else the alternating one
  const int n_xv = hpx * n_ent;
  const bool greedy = VARLEN && wpx <= 64 && n_xv <= kGreedyRounds * wpx;
  if constexpr (VARLEN || (CAUSAL && !LOCAL)) {
    const int n_x = hpx * (VARLEN ? n_ent : tm.n_qtiles);
    const int rounds = n_x / wpx, rem = n_x % wpx;
    n_items = rounds + (((rounds & 1) ? wpx - 1 - slot : slot) < rem ? 1 : 0);
  } else {
    n_items = max(0, min((tm.per_xcd - slot + wpx - 1) / wpx,
                         (tm.total - base_logical + wpx - 1) / wpx));
  }
  if (n_items == 0) return;

  const int Nq = p.Nq, Nk = p.Nk;
  const int off = Nk - Nq;   // the diagonal: key i + off for query i
  const int64_t ksn = p.k_sn * 2, vsn = p.v_sn * 2;  // row strides in bytes
  struct ItemBase {
    const uint8_t* q;   // row q0 + 32 * wave (clamped to the last row) of Q
    const uint8_t* k;   // key 0 of K
    const uint8_t* v;   // key 0 of V
    __bf16* o;          // row 0 of O
    float* lse;         // row 0 of LSE
    int q0;             // first query row of the tile
    int nt;             // key tiles it sees
    int kb;             // window: its first key tile
    int rot;            // window: step 0 visits key tile kb + rot
  };
  struct ItemSeq : ItemBase {
    int lq, lk;         // packed: the sequence's query rows and keys
    int kmin;           // packed: minus the sequence's first key
  };
  struct ItemBias : ItemSeq {
    const uint8_t* bias;  // bias: row min(q0 + 32 * wave, Nq - 1), key 0 of (batch, head)
    int brmax;            // bias: rows of this wavefront's block that exist, minus 1
  };
  using Item = std::conditional_t<BIAS, ItemBias, std::conditional_t<VARLEN, ItemSeq, ItemBase>>;
  auto item = [&](int it) {
    if constexpr (VARLEN) {
      Item r;
      // rank i of this XCD's (tile, head) list: the tile of rank i / hpx,
      // head xcd * hpx + i % hpx (the first item is rank `slot` in both deals)
      const int i = greedy ? (it == 0 ? slot : __builtin_amdgcn_readfirstlane(mine[it]))
                           : it * wpx + ((it & 1) ? wpx - 1 - slot : slot);
      const int e = __builtin_amdgcn_readfirstlane(ent[i / hpx]);
      const int b = e & 63, h = xcd * hpx + i % hpx;
      const int hk = h / p.head_group;
      const int4 sq = seq[b];
      const int2 sbb = sbase[b];
      const int q_lo = __builtin_amdgcn_readfirstlane(sbb.x), k_lo = __builtin_amdgcn_readfirstlane(sbb.y);
      r.lq = __builtin_amdgcn_readfirstlane(sq.x);
      r.lk = __builtin_amdgcn_readfirstlane(sq.y);
      r.kmin = -k_lo;
      r.q0 = (e >> 6) * kBr;
      r.kb = 0;
      r.rot = 0;
      // key tiles its rows see, made even and at least 2 (the extra tile,
      // placed inside the sequence's keys, is masked whole)
      const int kv = CAUSAL ? min(r.lk, min(r.q0 + kBr, r.lq) + (r.lk - r.lq)) : r.lk;
      const int nraw = (max(kv, 0) + kKT - 1) / kKT;
      r.nt = max(2, nraw + (nraw & 1));
      const int wrow = min(r.q0 + 32 * wave, r.lq - 1);
      // padded batches (BIAS): batch b at its batch strides (q_lo = k_lo = 0)
      const int64_t bb = BIAS ? (int64_t)b : (int64_t)0;
      r.q = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.q) + bb * p.q_sb +
                                                         h * p.q_sh + (int64_t)(q_lo + wrow) * p.q_sn));
      r.k = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.k) + bb * p.k_sb +
                                                         hk * p.k_sh + (int64_t)k_lo * p.k_sn));
      r.v = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.v) + bb * p.v_sb +
                                                         hk * p.v_sh + (int64_t)k_lo * p.v_sn));
      r.o = static_cast<__bf16*>(p.o) + bb * p.o_sb + (int64_t)q_lo * p.o_sn + h * p.o_sh;
      r.lse = p.lse + bb * p.l_sb + q_lo + h * p.l_sh;
      if constexpr (BIAS) {
        r.bias = uniform_ptr(reinterpret_cast<const uint8_t*>(p.bias + bb * p.bias_sb + h * p.bias_sh +
                                                              (int64_t)wrow * p.bias_sn));
        r.brmax = r.lq - 1 - wrow;
      }
      return r;
    }
    int qt, hb;
    if constexpr (CAUSAL && !LOCAL) {
      const int i = it * wpx + ((it & 1) ? wpx - 1 - slot : slot);
      qt = tm.n_qtiles - 1 - i / hpx;
      hb = xcd * hpx + i % hpx;
    } else {
      const int logical = base_logical + it * wpx;
      qt = logical % tm.n_qtiles;
      hb = logical / tm.n_qtiles;
    }
    const int h = hb % p.H, b = hb / p.H;
    const int hk = h / p.head_group;
    Item r;
    r.q0 = qt * kBr;
    r.nt = (CAUSAL ? min(Nk, r.q0 + kBr + off) : Nk) / kKT;
    r.kb = 0;
    r.rot = 0;
    if constexpr (LOCAL) {
      // key tiles from the left edge of its first row to the right edge of
      // its last, made even (one more whole tile, masked, on either side)
      int lo = max(r.q0 + off - p.win_left, 0) / kKT;
      int hi_t = min((r.q0 + kBr - 1 + off + p.win_right) / kKT + 1, Nk / kKT);
      if ((hi_t - lo) & 1) {
        if (lo > 0) --lo;
        else ++hi_t;   // hi_t odd < Nk / kKT, which is even
      }
      r.kb = lo;
      r.nt = hi_t - lo;
      // step t visits the tile whose absolute index is = t (mod nt): the
      // query tiles of one head on an XCD, all covering nt tiles, read the
      // same key tile at the same step (its later copies come from L2)
      r.rot = (r.nt - lo % r.nt) % r.nt;
    }
    const int wrow = min(r.q0 + 32 * wave, Nq - 1);
    r.q = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.q) + b * p.q_sb +
                                                       h * p.q_sh + (int64_t)wrow * p.q_sn));
    r.k = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.k) + b * p.k_sb +
                                                       hk * p.k_sh));
    r.v = uniform_ptr(reinterpret_cast<const uint8_t*>(static_cast<const __bf16*>(p.v) + b * p.v_sb +
                                                       hk * p.v_sh));
    r.o = static_cast<__bf16*>(p.o) + b * p.o_sb + h * p.o_sh;
    r.lse = p.lse + b * p.l_sb + h * p.l_sh;
    return r;
  };
  // key tile visited at step t of a query tile
  auto tix = [&](const Item& it, int t) {
    if constexpr (LOCAL) {
      const int x = t + it.rot;
      return it.kb + (x >= it.nt ? x - it.nt : x);
    } else {
      return t;
    }
  };
  // first key of the tile read at step t. Packed sequences: tile t holds
  // the sequence's keys [64 t, 64 t + 64) that exist; a tile reaching past
  // the last key is read shifted to end there (or, for a sequence of fewer
  // than 64 keys, to start at key 0 of the packed tensor), and the keys it
  // reads outside its own range are masked, so no copy leaves the tensors.
  // query rows of the tile's (batch, head) or sequence
  auto rows = [&](const Item& it) {
    if constexpr (VARLEN) return it.lq;
    else return Nq;
  };
  // Padded batches (BIAS) read tile t in place, or the last 64 keys of the
  // tensor when it reaches past them (a multiple of 4 keys: the bias
  // blocks' 16-byte chunks stay aligned).
  auto kpos = [&](const Item& it, int t) {
    if constexpr (BIAS) return min(kKT * t, Nk - kKT);
    else if constexpr (VARLEN) return max(min(kKT * t, it.lk - kKT), it.kmin);
    else return tix(it, t) * kKT;
  };

  uint8_t* const kbuf = smem;                    // K tile t in buffer t % 2
  uint8_t* const vbuf = smem + 2 * kKBytes;      // V tile t in buffer t % 2
  uint8_t* const qw = smem + kSmemKV + wave * kQWave;  // this wavefront's Q / O rows

  // ---- LDS DMA lane offsets of a full K / V tile (every tile is full here)
  uint32_t koff[kDmaPerWave], voff[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    koff[i] = (uint32_t)(k_dma_key<D, W>(wave, lane, i) * (int)ksn + k_dma_col<D, W>(wave, lane, i));
    voff[i] = (uint32_t)(v_dma_key<D, W>(wave, lane, i) * (int)vsn + v_dma_col<D, W>(wave, lane, i));
  }
  auto dma_k = [&](const uint8_t* tile, uint8_t* dst, int i) {
    dma16(tile, koff[i], dst + 1024 * (wave + W * i));
  };
  auto dma_v = [&](const uint8_t* tile, uint8_t* dst, int i) {
    dma16(tile, voff[i], dst + 1024 * (wave + W * i));
  };
  auto wait_tiles = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // ---- Q rows of this wavefront into its LDS rows: copy i holds rows
  // i * kRowsPerKB + lane / kC; the lane fetches chunk (lane % kC) ^ (row % kC)
  // of that row (rows past the last query re-read the last one).
  auto q_copy = [&](const Item& it, int i) {
    const int ln = fresh(lane);
    const int r = i * kRowsPerKB + ln / kC;
    const int wrow0 = it.q0 + 32 * wave;
    const int lq = rows(it);
    const int rel = max(min(wrow0 + r, lq - 1) - min(wrow0, lq - 1), 0);
    const int chunk = (ln % kC) ^ (r % kC);
    dma16(it.q, (uint32_t)(rel * (int)(p.q_sn * 2) + 16 * chunk), qw + 1024 * i);
  };
  // Q as the MFMA B operand: lane holds row l32, elements [16kk + 8hi, +8)
  bf16x8 qf[G::kNkk];
  // (addresses recomputed at each use: kept across the loop they would take
  // registers the loop needs)
  auto q_from_lds = [&]() {
    const int ln = fresh(lane);
    const uint8_t* const row = qw + (ln & 31) * kRowBytes;
    const int sw = (ln & 31) % kC, h = ln >> 5;
#pragma unroll
    for (int kk = 0; kk < G::kNkk; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(row + 16 * ((2 * kk + h) ^ sw));
  };

  // ---- MFMA operand addressing (as in the per-tile kernel)
  const uint8_t* const klane = kbuf + (l32 >> 4) * G::kKBlock + hi * 256 + (l32 & 15) * 16;
  const int gi = l32 & 15;
  const uint8_t* const vlane = vbuf + 2 * hi * G::kVBlock + 128 * (l32 >> 4) +
                               64 * ((gi >> 1) & 1) + 16 * (gi >> 2) + 8 * (gi & 1);
  // K fragment i of a tile: 32-key block i % NB, k-step i / NB
  constexpr int kNq = NB * G::kNkk;
  constexpr int kNv = 2 * NB * G::kNcb;
  auto kfrag = [&](const uint8_t* kb, int i) {
    return *reinterpret_cast<const bf16x8*>(kb + (i % NB) * 2 * G::kKBlock + (i / NB) * 512);
  };
  auto vfrag = [&](const uint8_t* vb, int i) {
    const uint8_t* p0 = vb + 4 * (i / G::kNcb) * G::kVBlock + 256 * (i % G::kNcb);
    return lds_read_tr_pair(p0, p0 + G::kVBlock);
  };

  f32x16 oacc[G::kNcb];
  float m_run = -INFINITY;  // reference R of this lane's row (base 2)
  float l_run = 0.f;
  // base-2 factor of the scores: scale * log2(e) on raw dot products, log2(e)
  // on biased scores (already scale * qk + bias)
  const float c2 = BIAS ? kLog2e : p.scale_log2;

  auto tile_max = [&](const f32x16 (&s)[NB]) {
    float m = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, s[bb][r]);
    return lane_pair_max(m) * c2;
  };
  auto exp_slice = [&](const f32x16 (&s)[NB], u32x4 (&pw)[NB][2], float m_use, float& rs, int i) {
    const int bb = i >> 3, r = 2 * (i & 7);
    float x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[bb][r + e], c2, -m_use));
      rs += x[e];
    }
    const bf16x2 v = {(__bf16)x[0], (__bf16)x[1]};
    uint32_t w = __builtin_bit_cast(uint32_t, v);
    asm volatile("" : "+v"(w), "+v"(rs));
    pw[bb][r >> 3][(r & 7) >> 1] = w;
  };

  // Software pipeline of one tile (see fwd_bf16_kernel.h): phase A = S_{j+1}
  // on the matrix pipe beside the second half of tile j's exponentials and
  // the tile copies; the overflow check; phase B = O += V_j P_j beside the
  // first half of tile j+1's exponentials.
  constexpr int kSlices = 8 * NB;
  constexpr int kPre = kSlices / 2;
  constexpr int kSlicesA = kSlices - kPre;
  constexpr int kNdma = 2 * kDmaPerWave;
  auto phase_a = [&](auto with_qk, const uint8_t* kb, const f32x16 (&sc)[NB], f32x16 (&sn)[NB],
                     u32x4 (&pb)[NB][2], float m_use, auto&& dma) {
    float rs = 0.f;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (decltype(with_qk)::value) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) sn[bb] = f32x16{};
      bf16x8 kf[kPf];
#pragma unroll
      for (int i = 0; i < kPf; ++i) kf[i] = kfrag(kb, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kNq; ++i) {
        sn[i % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % kPf], qf[i / NB], sn[i % NB], 0, 0, 0);
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
  auto phase_b = [&](auto with_next, const uint8_t* vb, u32x4 (&pb)[NB][2], const f32x16 (&sn)[NB],
                     float m_use, float& rs_next) {
    __builtin_amdgcn_s_setprio(0);
    bf16x8 vf[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) vf[i] = vfrag(vb, i);
    __builtin_amdgcn_sched_barrier(0);
    // the slices computed ahead write the P registers of key blocks
    // 0 .. NB/2 - 1 (16-key groups u < NB), read by MFMAs i < NB * kNcb
    constexpr int kPer = kSlices / kNv;
    constexpr int kB0 = kNv - kPre / kPer;
    static_assert(kPre % kPer == 0 && kB0 >= NB * G::kNcb, "slices must follow the MFMAs that read their P");
#pragma unroll
    for (int i = 0; i < kNv; ++i) {
      const int u = i / G::kNcb;
      oacc[i % G::kNcb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          vf[i % kPf], __builtin_bit_cast(bf16x8, pb[u >> 1][u & 1]), oacc[i % G::kNcb], 0, 0, 0);
      if (i + kPf < kNv) vf[i % kPf] = vfrag(vb, i + kPf);
      if constexpr (decltype(with_next)::value) {
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
  auto qk_plain = [&](const uint8_t* kb, f32x16 (&s)[NB]) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) s[bb] = f32x16{};
    bf16x8 kf[kPf];
#pragma unroll
    for (int i = 0; i < kPf; ++i) kf[i] = kfrag(kb, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kNq; ++i) {
      s[i % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % kPf], qf[i / NB], s[i % NB], 0, 0, 0);
      if (i + kPf < kNq) kf[i % kPf] = kfrag(kb, i + kPf);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // causal / window: the scores of key tile kv0.. of the tile at q0 hidden
  // from this lane's row become -inf (key > row + Nk - Nq + right, or, with a
  // window, key < row + Nk - Nq - left); only tiles crossing an edge of this
  // wavefront's rows (register r of block bb holds key kv0 + 32 bb +
  // 16 (r / 8) + 8 hi + r % 8)
  auto mask_causal = [&](f32x16 (&s)[NB], int q0, int kv0) {
    const int qmin = q0 + 32 * wave;
    const int offr = LOCAL ? off + p.win_right : off;
    const int offl = LOCAL ? off - p.win_left : 0;
    const bool right = kv0 + kKT - 1 > qmin + offr;
    const bool left = LOCAL && kv0 < qmin + 31 + offl;
    if (right || left) {
      const int row = qmin + l32;
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
          if (key > row + offr || (LOCAL && key < row + offl)) s[bb][r] = -INFINITY;
        }
    }
  };

  // packed sequences: the scores of tile t of `it` outside its own keys
  // [64 t, min(64 t + 64, keys)), or (causal) of keys past the row's
  // diagonal (key > row + keys - rows), become -inf
  auto mask_seq = [&](f32x16 (&s)[NB], const Item& it, int t) {
    if constexpr (VARLEN) {
      const int pos = kpos(it, t);
      const int klo = kKT * t, khi = min(klo + kKT, it.lk);
      const int qmin = it.q0 + 32 * wave;
      const int offr = it.lk - it.lq;
      const bool right = CAUSAL && pos + kKT - 1 > qmin + offr;
      if (pos < klo || pos + kKT > khi || right) {
        const int row = qmin + l32;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = pos + 32 * bb + 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key < klo || key >= khi || (CAUSAL && key > row + offr)) s[bb][r] = -INFINITY;
          }
      }
    }
  };

  // 1 KB piece i of the previous query tile's O, from this wavefront's LDS
  // rows to HBM (rows i * kRowsPerKB + lane / kC, whole 16-byte chunks)
  auto drain = [&](const Item& prv, int i) {
    const int ln = fresh(lane);
    const int r = i * kRowsPerKB + ln / kC;
    const u32x4 x = *reinterpret_cast<const u32x4*>(qw + 1024 * i + 16 * ln);
    const int row = prv.q0 + 32 * wave + r;
    if (row < rows(prv)) {
      const int chunk = (ln % kC) ^ (r % kC);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(prv.o + (int64_t)row * p.o_sn) + 16 * chunk) = x;
    }
  };

  // Bias blocks (BIAS): this wavefront's 32 rows x 64 keys of key tile t of
  // `it`, copied into its own 8 KB of LDS (chunk kc, keys 4 kc .. 4 kc + 3,
  // of row r at 16-byte slot 16 r + (kc ^ (r mod 16)): one row's 16 lanes
  // copy 256 contiguous bytes, and the reads below of 16 rows hit 16
  // different bank groups); rows past the last query re-read the last one.
  uint8_t* const bias_lds = smem + bias_lds_offset<D, NB>() + wave * kBiasWave;
  auto dma_bias = [&](const Item& it, int t) {
    if constexpr (BIAS) {
      const uint8_t* src = uniform_ptr(it.bias + 4 * kpos(it, t));
      const int ln = fresh(lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (ln >> 4);
        const int kc = (ln & 15) ^ (r & 15);
        dma16(src, (uint32_t)(min(r, it.brmax) * (int)(p.bias_sn * 4) + 16 * kc), bias_lds + 1024 * i);
      }
    }
  };
  // The block in LDS as 16-byte chunks of the lane's row: read g holds
  // chunk 8 (g / 4) + 4 ((g / 2) % 2) + 2 hi + g % 2, i.e. the keys of
  // registers 4 (g % 4) .. 4 (g % 4) + 3 of score block g / 4 (register r
  // of block bb holds key 32 bb + 16 (r / 8) + 8 hi + r % 8).
  auto bias_read = [&](int g) {
    const int kc = 8 * (g >> 2) + 4 * ((g >> 1) & 1) + 2 * hi + (g & 1);
    return *reinterpret_cast<const f32x4*>(bias_lds + 256 * l32 + 16 * (kc ^ (l32 & 15)));
  };
  // scores -> scale * qk + bias (natural units, one FMA); then, once this
  // wavefront's reads are done, the block of key tile t of `it` is copied
  // over the one just read
  auto add_bias = [&](f32x16 (&s)[NB], const Item& it, int t) {
    if constexpr (BIAS) {
      // vector memory operations complete in issue order: once at most the
      // kNdma K/V copies of this iteration's phase A are outstanding, the
      // block's copies (issued in the previous iteration, or the prologue)
      // and this iteration's O and Q copies have landed
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNdma) : "memory");
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const f32x4 x = bias_read(g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[g >> 2][4 * (g & 3) + e] = __builtin_fmaf(s[g >> 2][4 * (g & 3) + e], p.scale, x[e]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_bias(it, t);
    }
  };

  u32x4 pb[NB][2];
  float rs_half = 0.f;

  // Two kinds of iteration: ordinary (tile j+1 of the same query tile
  // follows) and the last of a query tile (its phase A computes the first
  // S^T of the tile `nxt`, with nxt's Q read from LDS, and its phase B
  // computes no exponentials ahead). The workgroup's very last query tile
  // ends the same way with nxt = itself (sixteen MFMAs and two tile copies
  // for nothing, once per workgroup: one code path fewer to fit in 256
  // registers).
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  auto iteration = [&](auto last, int j, const Item& cur, const Item& prv, const Item& nxt,
                       bool has_next, bool has_prev, f32x16 (&sc)[NB], f32x16 (&sn)[NB]) {
    constexpr bool kLast = decltype(last)::value;
    const int par = j & 1;
    if constexpr (!kLast) {
      // the previous query tile's O, from this wavefront's LDS rows to HBM
      // (two 1 KB row copies per iteration), then the next tile's Q rows
      // into the same LDS rows (one copy per iteration)
      if (has_prev && j < kDrainIters) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
          if (2 * j + c < kQCopies) drain(prv, 2 * j + c);
      }
      if (has_next && j >= kQ0 && j < kQ0 + kQCopies) q_copy(nxt, j - kQ0);
    } else {
      q_from_lds();   // nxt's Q (copied during this tile; own rows of Q)
    }
    // K_{j+2} and V_{j+1} of the stream into the buffers of K_j and V_{j-1};
    // past this query tile's keys they are nxt's first ones
    const int nt = cur.nt;
    auto ktile = [&](int t) {
      return t < nt ? cur.k + kpos(cur, t) * ksn : nxt.k + kpos(nxt, t - nt) * ksn;
    };
    auto vtile = [&](int t) {
      return t < nt ? cur.v + kpos(cur, t) * vsn : nxt.v + kpos(nxt, t - nt) * vsn;
    };
    const uint8_t* const kt = uniform_ptr(ktile(j + 2));
    const uint8_t* const vt = uniform_ptr(vtile(j + 1));
    uint8_t* const kd = kbuf + par * kKBytes;
    uint8_t* const vd = vbuf + (par ^ 1) * kKBytes;
    auto dma = [&](int s) {
#pragma unroll
      for (int n = 0; n < kNdma; ++n) {
        if ((n * kNq) / kNdma != s) continue;
        if (n < kDmaPerWave) dma_k(kt, kd, n);
        else dma_v(vt, vd, n - kDmaPerWave);
      }
    };
    float rs = rs_half + phase_a(Yes{}, klane + (par ^ 1) * kKBytes, sc, sn, pb,
                                 m_run == -INFINITY ? 0.f : m_run, dma);
    if (__builtin_amdgcn_ballot_w64(!(rs <= kBig) || m_run == -INFINITY) != 0) {
      // rare: move the reference to the tile maximum and redo the tile
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
    // S_{j+1}: key tile j + 1 of this query tile, or nxt's first. Bias: its
    // block (copied during the previous iteration) is added, then the block
    // of the tile after it (tile j + 2 of this query tile, else nxt's tile
    // j + 2 - nt) is copied over it once this wavefront's reads are done.
    if constexpr (BIAS) {
      if constexpr (kLast) add_bias(sn, nxt, 1);
      else if (j + 2 < nt) add_bias(sn, cur, j + 2);
      else add_bias(sn, nxt, 0);
    }
    if constexpr (VARLEN) {
      if constexpr (kLast) mask_seq(sn, nxt, 0);
      else mask_seq(sn, cur, j + 1);
    } else if constexpr (CAUSAL) {
      mask_causal(sn, kLast ? nxt.q0 : cur.q0, (kLast ? tix(nxt, 0) : tix(cur, j + 1)) * kKT);
    }
    using Next = std::integral_constant<bool, !kLast>;
    phase_b(Next{}, vlane + par * kKBytes, pb, sn, m_run == -INFINITY ? 0.f : m_run, rs_half);
    if constexpr (BIAS) {
      // the eight bias copies, this iteration's last vector memory
      // operations, may stay in flight into the next iteration; every K/V,
      // Q and O copy before them has landed
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
      wait_tiles();
    }
    __syncthreads();
  };

  // This wavefront's rows of the finished tile: O / l as bf16 into its LDS
  // rows, LSE straight to HBM.
  auto stage_o = [&](const Item& it) {
    const float l_tot = lane_pair_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const int ln = fresh(lane);
    uint8_t* const row = qw + (ln & 31) * kRowBytes + 8 * (ln >> 5);
    const int sw = (ln & 31) % kC;
#pragma unroll
    for (int cb = 0; cb < G::kNcb; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[cb][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(row + 16 * ((4 * cb + g) ^ sw)) = w;
      }
    const int my_q = it.q0 + 32 * wave + (ln & 31);
    if ((ln >> 5) == 0 && my_q < rows(it))
      it.lse[my_q] = (l_tot > 0.f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  };
  // the new query tile's first score tile: its reference and the
  // exponentials computed ahead of iteration 0
  auto start_tile = [&](const f32x16 (&s)[NB]) {
#pragma unroll
    for (int cb = 0; cb < G::kNcb; ++cb) oacc[cb] = f32x16{};
    l_run = 0.f;
    m_run = tile_max(s);
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    rs_half = 0.f;
#pragma unroll
    for (int k = 0; k < kPre; ++k) exp_slice(s, pb, m_use, rs_half, k);
  };

  f32x16 sa[NB], sb[NB];

  // ---- prologue of the first query tile
  {
    const Item c0 = item(0);
#pragma unroll
    for (int i = 0; i < kQCopies; ++i) q_copy(c0, i);
    dma_bias(c0, 0);
    const uint8_t* k0 = uniform_ptr(c0.k + kpos(c0, 0) * ksn);
    const uint8_t* v0 = uniform_ptr(c0.v + kpos(c0, 0) * vsn);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) dma_k(k0, kbuf, i);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) dma_v(v0, vbuf, i);
    const uint8_t* k1 = uniform_ptr(c0.k + kpos(c0, 1) * ksn);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) dma_k(k1, kbuf + kKBytes, i);
    if constexpr (VARLEN) {
      if (greedy && wave == 0) {
        // Greedy deal of this XCD's items (sorted longest first) while the
        // copies land: round r hands its wpx items, longest first, to the
        // workgroups in order of the work they hold (least first, ties by
        // slot). Lane s is workgroup slot s; every workgroup of the XCD
        // computes the same deal and keeps its own items.
        int load = 0, n_mine = 0;
        const int rounds = (n_xv + wpx - 1) / wpx;
        const int nk4 = (wpx + 3) >> 2;
        for (int r = 0; r < rounds; ++r) {
          const int ir = r * wpx + lane;   // the item of rank `lane` in this round
          const int c = (lane < wpx && ir < n_xv) ? icost[ir] : 0;
          const int key = lane < wpx ? (load << 6) | lane : 0x7fffffff;
          // every lane's key to LDS, then each lane counts the smaller ones
          // (one wavefront: its LDS accesses complete in order)
          gkey[lane] = key;
          int rank = 0;
#pragma unroll 4
          for (int q4 = 0; q4 < nk4; ++q4) {
            const int4 kk = reinterpret_cast<const int4*>(gkey)[q4];
            rank += (kk.x < key ? 1 : 0) + (kk.y < key ? 1 : 0) + (kk.z < key ? 1 : 0) + (kk.w < key ? 1 : 0);
          }
          const int ci = __builtin_amdgcn_ds_bpermute(rank << 2, c);
          const int ii = r * wpx + rank;
          if (lane < wpx && ii < n_xv) {
            load += ci;
            if (lane == slot) mine[n_mine] = ii;
            ++n_mine;
          }
        }
        if (lane == slot) mine[kGreedyRounds] = n_mine;
      }
    }
    // the Q rows and K_0 (the oldest copies; they complete in issue order):
    // V_0 and K_1 may land while S_0 is computed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerWave) : "memory");
    __syncthreads();
    if constexpr (VARLEN)
      if (greedy) n_items = __builtin_amdgcn_readfirstlane(mine[kGreedyRounds]);
    q_from_lds();
    qk_plain(klane, sa);
    add_bias(sa, c0, 1);
    if constexpr (VARLEN) mask_seq(sa, c0, 0);
    else if constexpr (CAUSAL) mask_causal(sa, c0.q0, tix(c0, 0) * kKT);
    // iteration 0 reads V_0 and K_1 and overwrites K buffer 0: every
    // wavefront's copies have landed and every one is done with K_0
    wait_tiles();
    __syncthreads();
    start_tile(sa);
  }

  for (int it = 0; it < n_items; ++it) {
    const bool has_next = it + 1 < n_items;
    const bool has_prev = it > 0;
    const Item cur = item(it);
    const Item prv = has_prev ? item(it - 1) : cur;
    const Item nxt = has_next ? item(it + 1) : cur;
    const int nt = cur.nt;
    // A causal query tile with too few key tiles to spread the previous O's
    // drain and the next Q's copy over its iterations does both here, at
    // its start (each drain's LDS read is complete before the copy that
    // overwrites its rows is issued: the store that uses it waits for it).
    bool spread_prev = has_prev, spread_next = has_next;
    if constexpr (CAUSAL || VARLEN) {
      if (nt < kQ0 + kQCopies + 1) {
        if (has_prev) {
#pragma unroll
          for (int i = 0; i < kQCopies; ++i) drain(prv, i);
        }
        if (has_next) {
#pragma unroll
          for (int i = 0; i < kQCopies; ++i) q_copy(nxt, i);
        }
        spread_prev = spread_next = false;
      }
    }
    for (int j = 0; j + 2 < nt; j += 2) {
      iteration(No{}, j, cur, prv, nxt, spread_next, spread_prev, sa, sb);
      iteration(No{}, j + 1, cur, prv, nxt, spread_next, spread_prev, sb, sa);
    }
    iteration(No{}, nt - 2, cur, prv, nxt, spread_next, spread_prev, sa, sb);
    // without a next query tile, nxt is this one: its Q rows are still in
    // LDS (nothing was copied over them) and its first S^T is computed again
    iteration(Yes{}, nt - 1, cur, prv, nxt, spread_next, spread_prev, sb, sa);
    // sa holds nxt's first S^T
    stage_o(cur);
    if (has_next) {
      start_tile(sa);
    } else {
      // no tile follows: copy O out at once (this wavefront's rows only)
#pragma unroll
      for (int i = 0; i < kQCopies; ++i) drain(cur, i);
    }
  }
  // the last bias copies must land in this workgroup's LDS before it ends
  if constexpr (BIAS) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, int NB, bool CAUSAL, bool LOCAL, bool VARLEN = false, bool BIAS = false>
hipError_t launch_stream_d(const FwdParams& p, const TileMap& tm, int grid, hipStream_t stream) {
  // K/V double buffers + Q/O rows (+ the packed sequences' tile list) (+ the
  // eight wavefronts' bias blocks)
  constexpr int kSmemAll = BIAS ? bias_lds_offset<D, NB>() + 8 * kBiasWave
                                : 4 * (32 * NB) * D * 2 + 8 * 32 * 2 * D + (VARLEN ? kSeqTableBytes : 0);
  static_assert(kSmemAll <= 160 * 1024, "LDS of one workgroup");
  static bool attr_set = false;  // benign race: every caller sets the same value
  auto kern = fwd_bf16_stream_kernel<D, NB, CAUSAL, LOCAL, VARLEN, BIAS>;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmemAll);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(512), kSmemAll, stream, p, tm);
  return hipGetLastError();
}

template <int D, int NB>
hipError_t launch_stream_mask(const FwdParams& p, const TileMap& tm, int grid, hipStream_t s) {
  return p.local ? launch_stream_d<D, NB, true, true>(p, tm, grid, s)
                 : p.causal ? launch_stream_d<D, NB, true, false>(p, tm, grid, s)
                            : launch_stream_d<D, NB, false, false>(p, tm, grid, s);
}

template <int D>
hipError_t launch_stream_varlen(const FwdParams& p, const TileMap& tm, int grid, hipStream_t s) {
  return p.causal ? launch_stream_d<D, 2, true, false, true>(p, tm, grid, s)
                  : launch_stream_d<D, 2, false, false, true>(p, tm, grid, s);
}

}  // namespace

hipError_t launch_bf16_stream(const FwdParams& p, const TileMap& tm, int d, int key_tile, int grid,
                              hipStream_t s) {
  if (p.bias != nullptr) {
    // padded batches with a bias: d = 64, 64-key tiles, not causal, bias
    // blocks by LDS DMA, B <= 64, B * n_qtiles query tiles per head at most
    // kMaxEntries
    if (d != 64 || key_tile != 64 || p.causal || p.local || p.cu_q != nullptr || p.n_split > 1 ||
        !p.bias_dma || p.B < 1 || p.B > kMaxSeqs || (int64_t)p.B * tm.n_qtiles > kMaxEntries ||
        p.H < 8 || p.H % 8 != 0 || p.Nk < 64)
      return hipErrorInvalidValue;
    return launch_stream_d<64, 2, false, false, true, true>(p, tm, grid, s);
  }
  if (p.cu_q != nullptr) {
    // packed sequences: 64-key tiles, no window, B <= 64, B * n_qtiles
    // query tiles per head at most kMaxEntries
    if (key_tile != 64 || p.local || p.B < 1 || p.B > kMaxSeqs ||
        (int64_t)p.B * tm.n_qtiles > kMaxEntries || p.H < 8 || p.H % 8 != 0 || p.Nk < 64)
      return hipErrorInvalidValue;
    if (d == 128) return launch_stream_varlen<128>(p, tm, grid, s);
    if (d == 64) return launch_stream_varlen<64>(p, tm, grid, s);
    return hipErrorInvalidValue;
  }
  if (d == 128 && key_tile == 64) return launch_stream_mask<128, 2>(p, tm, grid, s);
  if (d == 64 && key_tile == 64) return launch_stream_mask<64, 2>(p, tm, grid, s);
  if (d == 64 && key_tile == 128 && !p.causal) return launch_stream_d<64, 4, false, false>(p, tm, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
