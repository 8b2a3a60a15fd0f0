// C ABI front end: argument validation, error reporting and dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call never
// touches the device (and can be exercised on a machine without a GPU). The
// checks mirror the contract written in include/attn.h; the host-side checks
// that a kernel needs before launch (head dimension, dtype, last-dimension
// contiguity, output allocation) follow the C++ layer described in
// "flash-attention" (stanleyjacob.dev), Part IV, stage 3, except that here the
// caller allocates the outputs.

#include "attn.h"

#include <algorithm>
#include <cmath>
#include <tuple>
#include <utility>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "fwd_params.h"

namespace attn {
const char* hip_error_text(int code);  // runtime.hip
}

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

int64_t elem_bytes(int32_t dt) { return dt == ATTN_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks on a 4-D input/output view of dtype `dt`.
attn_status_t check_view(const char* name, const attn_tensor_t* t, int32_t dt) {
  if (t == nullptr) return fail(ATTN_ERR_INVALID, "%s: descriptor is NULL", name);
  for (int i = 0; i < 4; ++i) {
    if (t->shape[i] < 0) return fail(ATTN_ERR_INVALID, "%s: negative extent %lld in dim %d", name,
                                     (long long)t->shape[i], i);
    if (t->stride[i] < 0)
      return fail(ATTN_ERR_UNSUPPORTED, "%s: negative stride in dim %d", name, i);
  }
  if (t->dtype != dt)
    return fail(ATTN_ERR_INVALID, "%s: dtype %d, expected %d", name, (int)t->dtype, (int)dt);
  return ATTN_OK;
}

attn_status_t check_rows(const char* name, const attn_tensor_t* t) {
  // bf16 and f32 rows must start on 16-byte boundaries for vector loads
  const int64_t eb = elem_bytes(t->dtype);
  if (t->shape[3] > 1 && t->stride[3] != 1)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: last dimension must be contiguous (stride[3] == 1)", name);
  for (int i = 0; i < 3; ++i)
    if (t->shape[i] > 1 && (t->stride[i] * eb) % 16 != 0)
      return fail(ATTN_ERR_UNSUPPORTED, "%s: stride[%d] = %lld elements is not a multiple of 16 bytes",
                  name, i, (long long)t->stride[i]);
  if (!aligned16(t->data))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: data pointer is not 16-byte aligned", name);
  return ATTN_OK;
}

int64_t st(const attn_tensor_t* t, int i) { return t->shape[i] > 1 ? t->stride[i] : 0; }

constexpr int64_t kMaxExtent = (int64_t)1 << 30;

// Validates the arguments shared by every forward entry point and fills `p`.
// `empty` is set when there is nothing to write (B, H or Nq is 0).
attn_status_t prepare(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                      const attn_mask_t* bias_or_mask, int causal, float scale,
                      const attn_tensor_t* o, const attn_tensor_t* lse, attn::FwdParams& p,
                      bool& empty) {
  empty = false;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr)
    return fail(ATTN_ERR_INVALID, "q, k, v, o and lse descriptors must be non-NULL");
  const int32_t dt = q->dtype;
  if (dt != ATTN_BF16 && dt != ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "q: dtype %d is neither ATTN_BF16 nor ATTN_F32", (int)dt);
  attn_status_t s;
  if ((s = check_view("q", q, dt)) != ATTN_OK) return s;
  if ((s = check_view("k", k, dt)) != ATTN_OK) return s;
  if ((s = check_view("v", v, dt)) != ATTN_OK) return s;
  if ((s = check_view("o", o, dt)) != ATTN_OK) return s;
  if ((s = check_view("lse", lse, ATTN_F32)) != ATTN_OK) return s;

  const int64_t B = q->shape[0], H = q->shape[1], Nq = q->shape[2], d = q->shape[3];
  const int64_t Hk = k->shape[1], Nk = k->shape[2];
  if (k->shape[0] != B || v->shape[0] != B)
    return fail(ATTN_ERR_INVALID, "batch mismatch: q %lld, k %lld, v %lld", (long long)B,
                (long long)k->shape[0], (long long)v->shape[0]);
  if (v->shape[1] != Hk || v->shape[2] != Nk)
    return fail(ATTN_ERR_INVALID, "k and v must have the same [B, Hk, Nk] extents");
  if (k->shape[3] != d || v->shape[3] != d)
    return fail(ATTN_ERR_INVALID, "head dimension mismatch: q %lld, k %lld, v %lld", (long long)d,
                (long long)k->shape[3], (long long)v->shape[3]);
  if (o->shape[0] != B || o->shape[1] != H || o->shape[2] != Nq || o->shape[3] != d)
    return fail(ATTN_ERR_INVALID, "o must be [B, H, Nq, d] like q");
  if (lse->shape[0] != B || lse->shape[1] != H || lse->shape[2] != Nq || lse->shape[3] != 1)
    return fail(ATTN_ERR_INVALID, "lse must be [B, H, Nq, 1]");
  if (H > 0 && (Hk < 1 || H % Hk != 0))
    return fail(ATTN_ERR_INVALID, "key/value heads (%lld) must divide query heads (%lld)",
                (long long)Hk, (long long)H);
  // A NaN or infinite scale is malformed; a finite scale <= 0 is well formed
  // but outside what the kernels handle (they take the row maximum of the
  // raw dot products and scale it afterwards, which needs scale > 0).
  if (!std::isfinite(scale))
    return fail(ATTN_ERR_INVALID, "scale must be finite (got %g)", (double)scale);
  if (!(scale > 0.f))
    return fail(ATTN_ERR_UNSUPPORTED, "scale must be > 0 (got %g)", (double)scale);
  if (B > kMaxExtent || H > kMaxExtent || Nq > kMaxExtent || Nk > kMaxExtent)
    return fail(ATTN_ERR_UNSUPPORTED, "extents above 2^30 are not supported");
  if (d != 64 && d != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension %lld is not supported (64 or 128)", (long long)d);

  const attn_tensor_t* bias = bias_or_mask ? bias_or_mask->bias : nullptr;
  const int32_t* kv_len = bias_or_mask ? bias_or_mask->kv_len : nullptr;
  if (bias != nullptr) {
    if ((s = check_view("bias", bias, ATTN_F32)) != ATTN_OK) return s;
    if (!(bias->shape[0] == B || bias->shape[0] == 1) || !(bias->shape[1] == H || bias->shape[1] == 1) ||
        bias->shape[2] != Nq || bias->shape[3] != Nk)
      return fail(ATTN_ERR_INVALID, "bias must be [B|1, H|1, Nq, Nk]");
  }

  // empty work: nothing to write
  if (B == 0 || H == 0 || Nq == 0) {
    empty = true;
    return ATTN_OK;
  }

  if ((s = check_rows("q", q)) != ATTN_OK) return s;
  if ((s = check_rows("o", o)) != ATTN_OK) return s;
  if (Nk > 0) {
    if ((s = check_rows("k", k)) != ATTN_OK) return s;
    if ((s = check_rows("v", v)) != ATTN_OK) return s;
    // the kernels address the rows of one 64-key tile with 32-bit byte offsets
    const int64_t eb = dt == ATTN_BF16 ? 2 : 4;
    for (const attn_tensor_t* t : {k, v})
      if (Nk > 1 && 64 * t->stride[2] * eb >= (int64_t(1) << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: row stride %lld elements is too large (64 rows must span < 2 GiB)",
                    t == k ? "k" : "v", (long long)t->stride[2]);
  }
  if (lse->data == nullptr || (reinterpret_cast<uintptr_t>(lse->data) & 3u) != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "lse: data pointer is NULL or not 4-byte aligned");
  if (Nq > 1 && lse->stride[2] != 1)
    return fail(ATTN_ERR_UNSUPPORTED, "lse: rows must be contiguous (stride[2] == 1)");
  bool bias_vec = false;
  if (bias != nullptr && Nk > 0) {
    if (Nk > 1 && bias->stride[3] != 1)
      return fail(ATTN_ERR_UNSUPPORTED, "bias: last dimension must be contiguous (stride[3] == 1)");
    if (bias->data == nullptr || (reinterpret_cast<uintptr_t>(bias->data) & 3u) != 0)
      return fail(ATTN_ERR_UNSUPPORTED, "bias: data pointer is NULL or not 4-byte aligned");
    // rows that all start on 16-byte boundaries are read with vector loads
    bias_vec = aligned16(bias->data);
    for (int i = 0; i < 3; ++i)
      if (bias->shape[i] > 1 && bias->stride[i] % 4 != 0) bias_vec = false;
  }

  p = attn::FwdParams{};
  p.q = q->data;
  p.k = k->data;
  p.v = v->data;
  p.o = o->data;
  p.lse = static_cast<float*>(lse->data);
  p.bias = bias ? static_cast<const float*>(bias->data) : nullptr;
  p.kv_len = kv_len;
  p.q_sb = st(q, 0); p.q_sh = st(q, 1); p.q_sn = st(q, 2);
  p.k_sb = st(k, 0); p.k_sh = st(k, 1); p.k_sn = st(k, 2);
  p.v_sb = st(v, 0); p.v_sh = st(v, 1); p.v_sn = st(v, 2);
  p.o_sb = st(o, 0); p.o_sh = st(o, 1); p.o_sn = st(o, 2);
  p.l_sb = st(lse, 0); p.l_sh = st(lse, 1);
  if (bias) {
    p.bias_sb = st(bias, 0);
    p.bias_sh = st(bias, 1);
    p.bias_sn = st(bias, 2);
  }
  p.B = (int32_t)B;
  p.H = (int32_t)H;
  p.Hk = (int32_t)Hk;
  p.Nq = (int32_t)Nq;
  p.Nk = (int32_t)Nk;
  p.head_group = (int32_t)(H / Hk);
  p.causal = causal ? 1 : 0;
  p.bias_vec = bias_vec ? 1 : 0;
  p.scale_log2 = scale * 1.44269504088896341f;
  p.scale = scale;
  p.n_split = 1;
  p.pack = 1;

  // Mask kind: none, causal (a window with right bound 0 and no left
  // bound), or a general window, launched on the causal instantiations with
  // both bounds clamped to values that exclude nothing more than intended.
  const bool win = bias_or_mask != nullptr && bias_or_mask->window != 0;
  int64_t wl = win ? bias_or_mask->window_left : -1;
  int64_t wr = win ? bias_or_mask->window_right : -1;
  if (causal) wr = 0;
  if (wl >= 0 || wr > 0) {
    p.causal = 1;
    p.local = 1;
    p.win_left = (int32_t)(wl < 0 ? Nk : std::min<int64_t>(wl, Nk));
    p.win_right = (int32_t)(wr < 0 ? Nq : std::min<int64_t>(wr, Nq));
  } else {
    p.causal = wr == 0 ? 1 : 0;
  }

  // grid size: 8 * ceil(B*H*ceil(Nq/16)/8) workgroups at most (f32 tiles are smallest)
  const int64_t tiles = B * H * ((Nq + 15) / 16);
  if (tiles > ((int64_t)1 << 31) - 64)
    return fail(ATTN_ERR_UNSUPPORTED, "problem needs more than 2^31 workgroups");
  return ATTN_OK;
}

attn_status_t launch(const attn::FwdParams& p, int32_t dt, int d, void* stream) {
  const int rc = (dt == ATTN_BF16) ? attn::launch_fwd_bf16(p, d, stream)
                                   : attn::launch_fwd_f32(p, d, stream);
  if (rc != 0) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", attn::hip_error_text(rc));
  return ATTN_OK;
}

// Keys per split for a requested split count: a whole number of 64-key tiles.
int64_t split_keys(int64_t Nk, int64_t num_splits) {
  const int64_t per = (Nk + num_splits - 1) / num_splits;
  return (per + 63) / 64 * 64;
}

constexpr int kMaxSplits = 1024;

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

attn_status_t attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                       const attn_mask_t* bias_or_mask, int causal, float scale,
                       const attn_tensor_t* o, const attn_tensor_t* lse, void* stream) {
  g_last_error.clear();
  attn::FwdParams p;
  bool empty;
  attn_status_t s = prepare(q, k, v, bias_or_mask, causal, scale, o, lse, p, empty);
  if (s != ATTN_OK || empty) return s;
  return launch(p, q->dtype, (int)q->shape[3], stream);
}

int64_t attn_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t d,
                                        int32_t num_splits) {
  if (B < 0 || H < 0 || Nq < 0 || d < 0 || num_splits < 1) return -1;
  if (B > kMaxExtent || H > kMaxExtent || Nq > kMaxExtent || d > 1024 || num_splits > kMaxSplits)
    return -1;
  // partial outputs [num_splits, B, H, Nq, d] then log-sum-exps [num_splits, B, H, Nq], fp32
  const double bytes = (double)num_splits * B * H * Nq * (d + 1) * 4.0;
  if (bytes > 9.0e18) return -1;
  return (int64_t)num_splits * B * H * Nq * (d + 1) * 4;
}

int32_t attn_fwd_splitkv_num_splits(int64_t B, int64_t H, int64_t Hk, int64_t Nq, int64_t Nk,
                                    int64_t d, int causal, int has_bias) {
  if (B <= 0 || H <= 0 || Hk <= 0 || H % Hk != 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128))
    return 1;
  // Workgroups without a split, against the 512 that MI355X runs at once
  // (256 CUs, two workgroups each): aim for one full round of workgroups,
  // with at least 256 keys (four tiles) per split. (Measured on the decoding
  // workloads: one round beats two; fewer splits leave CUs idle.)
  const int pack = attn::fwd_bf16_pack(H / Hk, Nq);
  const int64_t nrows = pack * Nq;
  const int64_t rows = attn::fwd_bf16_rows((int)d, nrows, causal != 0, has_bias != 0, true);
  const int64_t wgs = B * (H / pack) * ((nrows + rows - 1) / rows);
  constexpr int64_t kTarget = 512;
  int64_t n = (kTarget + wgs - 1) / wgs;
  n = std::min<int64_t>(n, std::max<int64_t>(1, Nk / 256));
  n = std::min<int64_t>(n, kMaxSplits);
  return (int32_t)std::max<int64_t>(n, 1);
}

}  // extern "C"

namespace {

// The split-key forward with its partials in `workspace` (the caller's, or,
// noalloc, this device's scratch array, fetched only once every argument
// has been checked and a split is needed).
attn_status_t splitkv(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                      const attn_mask_t* bias_or_mask, int causal, float scale,
                      int32_t num_splits, void* workspace, int64_t workspace_bytes, bool noalloc,
                      const attn_tensor_t* o, const attn_tensor_t* lse, void* stream) {
  g_last_error.clear();
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(ATTN_ERR_INVALID, "num_splits must be in [1, %d] (got %d)", kMaxSplits, (int)num_splits);
  attn::FwdParams p;
  bool empty;
  attn_status_t s = prepare(q, k, v, bias_or_mask, causal, scale, o, lse, p, empty);
  if (s != ATTN_OK || empty) return s;
  if (q->dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "the split-key forward supports bf16 only");
  const int d = (int)q->shape[3];
  const int64_t kv_split = p.Nk > 0 ? split_keys(p.Nk, num_splits) : 64;
  const int64_t n_split = p.Nk > 0 ? (p.Nk + kv_split - 1) / kv_split : 1;
  // a single split is the plain forward: no workspace is used
  if (n_split <= 1) return launch(p, ATTN_BF16, d, stream);

  const int64_t need = attn_fwd_splitkv_workspace_size(p.B, p.H, p.Nq, d, (int32_t)n_split);
  if (need < 0) return fail(ATTN_ERR_UNSUPPORTED, "workspace size overflows");
  if (noalloc) {
    if (need > attn::kNoallocScratchBytes)
      return fail(ATTN_ERR_UNSUPPORTED,
                  "%lld splits of this shape need %lld bytes of partials, more than the %lld-byte "
                  "device scratch of the no-allocation entry point (use fewer splits, or "
                  "attn_fwd_splitkv with a workspace)",
                  (long long)n_split, (long long)need, (long long)attn::kNoallocScratchBytes);
  } else {
    if (workspace == nullptr || !aligned16(workspace))
      return fail(ATTN_ERR_INVALID, "workspace is NULL or not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(ATTN_ERR_INVALID, "workspace of %lld bytes is too small (%lld needed for %lld splits)",
                  (long long)workspace_bytes, (long long)need, (long long)n_split);
  }
  const int pack = attn::fwd_bf16_pack(p.head_group, p.Nq);
  const int64_t nrows = (int64_t)pack * p.Nq;
  const int rows = attn::fwd_bf16_rows(d, nrows, p.causal != 0, p.bias != nullptr, true);
  const int64_t wgs = (int64_t)p.B * (p.H / pack) * ((nrows + rows - 1) / rows) * n_split;
  if (wgs > ((int64_t)1 << 31) - 64 || (int64_t)p.B * p.H * p.Nq > ((int64_t)1 << 32))
    return fail(ATTN_ERR_UNSUPPORTED, "problem needs more than 2^31 workgroups");
  if (noalloc) {
    const int rc = attn::noalloc_scratch(&workspace);
    if (rc != 0)
      return fail(ATTN_ERR_HIP, "device scratch address unavailable: %s", attn::hip_error_text(rc));
  }

  p.kv_split = (int32_t)kv_split;
  p.n_split = (int32_t)n_split;
  p.pack = pack;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + n_split * (int64_t)p.B * p.H * p.Nq * d;
  int rc = attn::launch_fwd_bf16(p, d, stream);
  if (rc == 0) rc = attn::launch_combine_bf16(p, d, stream);
  if (rc != 0) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", attn::hip_error_text(rc));
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_splitkv(const attn_tensor_t* q, const attn_tensor_t* k,
                               const attn_tensor_t* v, const attn_mask_t* bias_or_mask,
                               int causal, float scale, int32_t num_splits, void* workspace,
                               int64_t workspace_bytes, const attn_tensor_t* o,
                               const attn_tensor_t* lse, void* stream) {
  return splitkv(q, k, v, bias_or_mask, causal, scale, num_splits, workspace, workspace_bytes,
                 false, o, lse, stream);
}

attn_status_t attn_fwd_splitkv_noalloc(const attn_tensor_t* q, const attn_tensor_t* k,
                                       const attn_tensor_t* v, const attn_mask_t* bias_or_mask,
                                       int causal, float scale, int32_t num_splits,
                                       const attn_tensor_t* o, const attn_tensor_t* lse,
                                       void* stream) {
  return splitkv(q, k, v, bias_or_mask, causal, scale, num_splits, nullptr, 0, true, o, lse,
                 stream);
}

attn_status_t attn_fwd_varlen(const attn_tensor_t* q, const attn_tensor_t* k,
                              const attn_tensor_t* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                              const attn_mask_t* window_mask, int causal, float scale,
                              const attn_tensor_t* o, const attn_tensor_t* lse, void* stream) {
  g_last_error.clear();
  if (window_mask != nullptr && (window_mask->bias != nullptr || window_mask->kv_len != nullptr))
    return fail(ATTN_ERR_INVALID, "packed sequences take no bias or kv_len (their lengths are "
                                  "the offsets)");
  for (const attn_tensor_t* t : {q, k, v, o, lse})
    if (t != nullptr && t->shape[0] != 1)
      return fail(ATTN_ERR_INVALID, "packed tensors are [1, heads, total rows, d] (got %lld in dim 0)",
                  (long long)t->shape[0]);
  if (num_seqs < 0 || max_seqlen_q < 0)
    return fail(ATTN_ERR_INVALID, "num_seqs and max_seqlen_q must be >= 0");
  attn::FwdParams p;
  bool empty;
  attn_status_t s = prepare(q, k, v, window_mask, causal, scale, o, lse, p, empty);
  if (s != ATTN_OK || empty) return s;
  if (num_seqs == 0 || max_seqlen_q == 0) return ATTN_OK;
  for (const int32_t* cu : {cu_seqlens_q, cu_seqlens_k})
    if (cu == nullptr || (reinterpret_cast<uintptr_t>(cu) & 3u) != 0)
      return fail(ATTN_ERR_INVALID, "cu_seqlens_q and cu_seqlens_k must be non-NULL, 4-byte aligned");
  const int64_t max_q = std::min<int64_t>(max_seqlen_q, p.Nq);
  if ((int64_t)num_seqs * p.H * ((max_q + 15) / 16) > ((int64_t)1 << 31) - 64)
    return fail(ATTN_ERR_UNSUPPORTED, "problem needs more than 2^31 workgroups");
  p.B = num_seqs;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.max_q = (int32_t)max_q;
  p.q_sb = p.k_sb = p.v_sb = p.o_sb = p.l_sb = 0;
  return launch(p, q->dtype, (int)q->shape[3], stream);
}

int64_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq) {
  if (B < 0 || H < 0 || Nq < 0 || B > kMaxExtent || H > kMaxExtent || Nq > kMaxExtent) return -1;
  const double bytes = 8.0 * (double)B * (double)H * (double)Nq;
  if (bytes > 9.0e18) return -1;
  return 8 * B * H * Nq;  // D and the base-2 log-sum-exp, fp32, per query row
}

attn_status_t attn_bwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                       const attn_tensor_t* o, const attn_tensor_t* lse,
                       const attn_tensor_t* dout, const attn_mask_t* bias_or_mask, int causal,
                       float scale, void* workspace, int64_t workspace_bytes,
                       const attn_tensor_t* dq, const attn_tensor_t* dk,
                       const attn_tensor_t* dv, void* stream) {
  g_last_error.clear();
  // the forward's own checks cover q, k, v, o, lse, the mask and the scale
  attn::FwdParams f;
  bool empty;
  attn_status_t s = prepare(q, k, v, bias_or_mask, causal, scale, o, lse, f, empty);
  if (s != ATTN_OK) return s;
  if (q->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the backward supports bf16 only");
  if (dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(ATTN_ERR_INVALID, "dout, dq, dk and dv descriptors must be non-NULL");
  for (auto [name, t, ref] : {std::tuple{"dout", dout, q}, std::tuple{"dq", dq, q},
                               std::tuple{"dk", dk, k}, std::tuple{"dv", dv, v}}) {
    if ((s = check_view(name, t, ATTN_BF16)) != ATTN_OK) return s;
    for (int i = 0; i < 4; ++i)
      if (t->shape[i] != ref->shape[i])
        return fail(ATTN_ERR_INVALID, "%s must have the shape of %s", name, ref == q ? "q" : "k / v");
  }
  if (empty) {
    // B, H or Nq is 0: no query sees any key, so dK = dV = 0 wherever there
    // are keys (H = 0 with Hk > 0, or Nq = 0 with Nk > 0)
    const int64_t B = k->shape[0], Hk = k->shape[1], Nk = k->shape[2], d = k->shape[3];
    if (B == 0 || Hk == 0 || Nk == 0) return ATTN_OK;
    for (auto [name, t] : {std::pair{"dk", dk}, std::pair{"dv", dv}})
      if ((s = check_rows(name, t)) != ATTN_OK) return s;
    for (const attn_tensor_t* t : {dk, dv}) {
      const int rc = attn::launch_zero_bf16(t->data, B, Hk, Nk, (int)d, st(t, 0), st(t, 1),
                                            st(t, 2), stream);
      if (rc != 0) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", attn::hip_error_text(rc));
    }
    return ATTN_OK;
  }
  for (auto [name, t] : {std::pair{"dout", dout}, std::pair{"dq", dq}})
    if ((s = check_rows(name, t)) != ATTN_OK) return s;
  // the dK/dV kernel streams 64-row tiles of q and dout, addressing their
  // rows with 32-bit byte offsets
  for (auto [name, t] : {std::pair{"q", q}, std::pair{"dout", dout}})
    if (f.Nq > 1 && 64 * t->stride[2] * 2 >= (int64_t(1) << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "%s: row stride %lld elements is too large (64 rows must span < 2 GiB)",
                  name, (long long)t->stride[2]);
  if (f.Nk > 0)
    for (auto [name, t] : {std::pair{"dk", dk}, std::pair{"dv", dv}})
      if ((s = check_rows(name, t)) != ATTN_OK) return s;
  const int64_t need = attn_bwd_workspace_size(f.B, f.H, f.Nq);
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(ATTN_ERR_INVALID, "workspace is NULL or not 16-byte aligned");
  if (need < 0 || workspace_bytes < need)
    return fail(ATTN_ERR_INVALID, "workspace of %lld bytes is too small (%lld needed)",
                (long long)workspace_bytes, (long long)need);

  attn::BwdParams p{};
  p.q = f.q; p.k = f.k; p.v = f.v; p.o = f.o; p.lse = f.lse;
  p.do_ = dout->data;
  p.dq = dq->data; p.dk = dk->data; p.dv = dv->data;
  p.bias = f.bias; p.kv_len = f.kv_len;
  p.dsum = static_cast<float*>(workspace);
  p.lse2 = p.dsum + (int64_t)f.B * f.H * f.Nq;
  p.q_sb = f.q_sb; p.q_sh = f.q_sh; p.q_sn = f.q_sn;
  p.k_sb = f.k_sb; p.k_sh = f.k_sh; p.k_sn = f.k_sn;
  p.v_sb = f.v_sb; p.v_sh = f.v_sh; p.v_sn = f.v_sn;
  p.o_sb = f.o_sb; p.o_sh = f.o_sh; p.o_sn = f.o_sn;
  p.do_sb = st(dout, 0); p.do_sh = st(dout, 1); p.do_sn = st(dout, 2);
  p.dq_sb = st(dq, 0); p.dq_sh = st(dq, 1); p.dq_sn = st(dq, 2);
  p.dk_sb = st(dk, 0); p.dk_sh = st(dk, 1); p.dk_sn = st(dk, 2);
  p.dv_sb = st(dv, 0); p.dv_sh = st(dv, 1); p.dv_sn = st(dv, 2);
  p.l_sb = f.l_sb; p.l_sh = f.l_sh;
  p.bias_sb = f.bias_sb; p.bias_sh = f.bias_sh; p.bias_sn = f.bias_sn;
  p.B = f.B; p.H = f.H; p.Hk = f.Hk; p.Nq = f.Nq; p.Nk = f.Nk;
  p.head_group = f.head_group;
  p.causal = f.causal; p.local = f.local;
  p.win_left = f.win_left; p.win_right = f.win_right;
  p.scale = scale;
  p.scale_log2 = f.scale_log2;
  const int rc = attn::launch_bwd_bf16(p, (int)q->shape[3], stream);
  if (rc != 0) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", attn::hip_error_text(rc));
  return ATTN_OK;
}

}  // extern "C"
