/*
 * attn.h - C ABI of the fused exact attention forward for AMD Instinct MI355X
 * (gfx950).
 *
 * The library computes, for every batch entry b and head h,
 *
 *     S = scale * Q K^T + Bias,   O = softmax_row(S) V,
 *     LSE_i = log( sum_j exp(S_ij) )          (natural logarithm)
 *
 * without ever writing S or P = softmax_row(S) to device memory: each
 * workgroup owns a tile of query rows and streams key/value tiles through LDS,
 * folding each score tile into a running row maximum m, a running denominator
 * l and an unnormalised output accumulator, rescaled whenever the maximum
 * grows, and divides once at the end.
 *
 * Definitions followed:
 *   - the function: "Understanding FlashAttention Pt 1: Personal Notes",
 *     section 0.2 "Notation" (S = QK^T/sqrt(d) + B, P = softmax_row(S), O = PV);
 *   - the streaming recurrence: same page, sections 2.3 and 2.4 (online
 *     softmax and the blockwise merge recurrence);
 *   - the tiled forward with query tiles outermost: same page, section 3.1,
 *     and "FlashAttention: Mathematical Foundations, Online Softmax Tiling,
 *     IO-Awareness, and Exact Attention Scaling", section 5 (loop order);
 *   - masks and tile skipping: first page, section 3.5;
 *   - the LSE output, scale folding into base-2 exponentials and the
 *     fully-masked-row rule: "flash-attention" (stanleyjacob.dev), Parts IV
 *     (stages 5-7) and VI, and its answer Q10 for causal alignment.
 *
 * Conventions
 *   - All tensor data pointers are DEVICE pointers. Strides are in elements.
 *   - Layout is [B, H, N, d] (batch, head, sequence, head dimension).
 *   - Ownership: the caller allocates every buffer and keeps ownership. The
 *     library allocates no device memory and keeps no pointer after a call.
 *   - Asynchrony: attn_fwd validates its arguments on the host, enqueues one
 *     kernel on `stream` and returns. ATTN_OK means "enqueued"; a device-side
 *     fault surfaces at the caller's next synchronisation.
 *   - Errors: a non-OK status means nothing was enqueued and no output byte
 *     was written; attn_last_error() then returns a description. No C++
 *     exception crosses this interface.
 *   - Thread safety: calls are reentrant and may be made from several host
 *     threads; the error text is kept per thread.
 */
#ifndef EXACT_IO_AWARE_06_AMD_ATTN_H
#define EXACT_IO_AWARE_06_AMD_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 6

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* malformed arguments: null pointer, shape mismatch, NaN or infinite scale */
  ATTN_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle (head dim, dtype, stride, alignment, scale <= 0) */
  ATTN_ERR_HIP = 3          /* the HIP runtime refused the launch; see attn_last_error() */
} attn_status_t;

typedef enum {
  ATTN_BF16 = 0, /* bfloat16 storage */
  ATTN_F32 = 1   /* IEEE binary32 storage */
} attn_dtype_t;

/* A strided 4-D view of device memory. */
typedef struct {
  void* data;          /* device pointer to element [0,0,0,0] */
  int32_t dtype;       /* an attn_dtype_t value */
  int64_t shape[4];
  int64_t stride[4];   /* in elements; stride[3] must be 1 */
} attn_tensor_t;

/* Optional terms on the scores. A zero-initialised struct adds nothing. */
typedef struct {
  /* NULL, or float32 [B|1, H|1, Nq, Nk]: added to scale*QK^T (it is NOT
     multiplied by `scale`). A dimension of extent 1 is broadcast (its stride
     is ignored). stride[3] must be 1 and data 4-byte aligned; rows that start
     on 16-byte boundaries (16-byte aligned data, strides multiples of 4) are
     read with wider loads. -inf entries are allowed and remove the pair. */
  const attn_tensor_t* bias;
  /* NULL, or a DEVICE pointer to int32[B]: key j of batch entry b takes part
     only if j < kv_len[b] (values are clamped to [0, Nk]); the same as an
     additive -inf bias on the padded keys. */
  const int32_t* kv_len;
  /* Sliding window (local attention), used when `window` is non-zero: key j
     takes part for query i only if
         i + (Nk - Nq) - window_left <= j <= i + (Nk - Nq) + window_right,
     the band around the bottom-right-aligned diagonal; a negative bound
     leaves that side open. `causal` != 0 sets window_right to 0 whatever
     its value. Whole key tiles outside the band are skipped. ("Understanding
     FlashAttention Pt 1", section 3.5, connection to local attention;
     "FlashAttention, Explained", section 14, sliding-window masks skip
     every tile outside the band; "flash-attention", Part III, window_size.) */
  int32_t window;
  int32_t window_left;
  int32_t window_right;
} attn_mask_t;

/*
 * attn_fwd - enqueue the attention forward on `stream`.
 *
 *   q    [B, H,  Nq, d]  bf16 or f32
 *   k    [B, Hk, Nk, d]  same dtype as q; Hk divides H (query head h reads
 *                        key/value head h / (H / Hk); Hk == H is plain
 *                        multi-head attention)
 *   v    [B, Hk, Nk, d]  same dtype as q
 *   bias_or_mask         NULL, or the optional terms above
 *   causal               non-zero: key j is hidden from query i when
 *                        j > i + (Nk - Nq) (aligned to the bottom-right
 *                        corner, so the last query sees every key)
 *   scale                multiplies QK^T (callers usually pass 1/sqrt(d)); a
 *                        NaN or infinite scale is ATTN_ERR_INVALID, a finite
 *                        scale <= 0 ATTN_ERR_UNSUPPORTED (the kernels scale
 *                        the row maximum of the raw dot products)
 *   o    [B, H,  Nq, d]  output, same dtype as q
 *   lse  [B, H,  Nq, 1]  output, float32; stride[2] must be 1
 *   stream               a hipStream_t, or NULL for the default stream
 *
 * Supported: d in {64, 128}; dtype bf16 or f32; stride[3] == 1 for q, k, v,
 * o; data pointers 16-byte aligned and strides of dimensions 0-2 multiples of
 * 16 bytes. Negative strides are not supported. The row stride of k and v
 * (stride[2]) times 64 rows must span less than 2 GiB. o and lse must not
 * overlap the inputs or each other.
 *
 * A row whose keys are all masked gets O = 0 and LSE = -inf. B, H or Nq equal
 * to 0 is a no-op that returns ATTN_OK; Nk == 0 writes O = 0 and LSE = -inf.
 */
attn_status_t attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k,
                       const attn_tensor_t* v, const attn_mask_t* bias_or_mask,
                       int causal, float scale, const attn_tensor_t* o,
                       const attn_tensor_t* lse, void* stream);

/*
 * Split-key forward (flash-decoding).
 *
 * Same function and outputs as attn_fwd, for shapes with few query rows per
 * (batch, head) - decoding, Nq = 1 - where one workgroup per query tile
 * leaves most compute units idle. The keys are cut into splits of whole
 * 64-key tiles; each workgroup computes one query tile against one split and
 * writes that split's normalised output O_s and log-sum-exp LSE_s (fp32) to
 * the workspace; a second kernel merges the splits with the log-sum-exp
 * identity of the blockwise softmax:
 *
 *     M = max_s LSE_s,  w_s = exp(LSE_s - M),
 *     O = sum_s w_s O_s / sum_s w_s,  LSE = M + log(sum_s w_s).
 *
 * Definitions followed: "Understanding FlashAttention Pt 1: Personal Notes",
 * section 2.4 (merging two softmax blocks); "FlashAttention: Mathematical
 * Foundations, Online Softmax Tiling, IO-Awareness, and Exact Attention
 * Scaling", section 7 (flash-decoding: split the keys, reduce with the LSE);
 * "FlashAttention, Explained", section 25.
 */

/* Bytes of workspace attn_fwd_splitkv needs for num_splits splits of a
   [B, H, Nq, d] problem: num_splits * B * H * Nq * (d + 1) * 4. Returns -1
   for a negative extent, num_splits outside [1, 1024] or d above 1024. */
int64_t attn_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t d,
                                        int32_t num_splits);

/* A split count for this shape on MI355X (H query heads, Hk key/value
   heads): enough splits for one round of workgroups on its 256 compute
   units (two per unit), with at least 256 keys per split, at most 1024. Returns 1
   (no split) when splitting does not help or the shape is empty or
   unsupported. A host-only computation. */
int32_t attn_fwd_splitkv_num_splits(int64_t B, int64_t H, int64_t Hk, int64_t Nq, int64_t Nk,
                                    int64_t d, int causal, int has_bias);

/*
 * attn_fwd_splitkv - enqueue the split-key forward on `stream`.
 *
 * Arguments q, k, v, bias_or_mask, causal, scale, o, lse and stream are as
 * for attn_fwd, with the same checks, except that only bf16 is supported.
 *
 *   num_splits       requested number of splits, in [1, 1024]. The keys are
 *                    cut into ceil(Nk / S) splits of S keys, S =
 *                    ceil(Nk / num_splits) rounded up to a multiple of 64, so
 *                    fewer splits may be used. With one split the call is
 *                    exactly attn_fwd and the workspace is not touched.
 *   workspace        DEVICE pointer, 16-byte aligned, owned by the caller,
 *                    used as scratch by the two kernels of this call: its
 *                    contents on entry are ignored and on return undefined.
 *                    It must not overlap any tensor of the call, and calls
 *                    that run concurrently need distinct workspaces.
 *   workspace_bytes  at least attn_fwd_splitkv_workspace_size(B, H, Nq, d,
 *                    num_splits) (checked against the split count used).
 *
 * With grouped key/value heads (Hk < H) and Nq <= 64, the H / Hk query
 * heads that share a key/value head are computed by the same workgroups, so
 * K and V are read once per key/value head rather than once per query head.
 *
 * Enqueues two kernels (the split forward, then the merge) and returns; the
 * error behaviour is that of attn_fwd. Results agree with attn_fwd up to
 * rounding: the splits' outputs are kept in fp32 and rounded to bf16 once,
 * after the merge.
 */
attn_status_t attn_fwd_splitkv(const attn_tensor_t* q, const attn_tensor_t* k,
                               const attn_tensor_t* v, const attn_mask_t* bias_or_mask,
                               int causal, float scale, int32_t num_splits, void* workspace,
                               int64_t workspace_bytes, const attn_tensor_t* o,
                               const attn_tensor_t* lse, void* stream);

/*
 * attn_fwd_splitkv_noalloc - attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, function, checks and results as attn_fwd_splitkv, without
 * the workspace: the split partials go to a file-scope device array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library. This call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); on its
 * first call on a device (the calling thread's current device, which must
 * hold the tensors and own `stream`) it looks up that device's copy of the
 * array once. Each device keeps its copy until the process ends.
 *
 *   - A split count whose partials need more than ATTN_NOALLOC_SCRATCH_BYTES
 *     (num_splits * B * H * Nq * (d + 1) * 4 for the splits used) returns
 *     ATTN_ERR_UNSUPPORTED before anything is enqueued.
 *   - Every call on one device shares that device's array, and nothing in
 *     it has to start at zero (each call writes every partial it reads).
 *     Calls whose kernels can overlap on one device - on different streams,
 *     or from several host threads - race on it: serialise them (one
 *     stream), or use attn_fwd_splitkv with distinct workspaces.
 *   - With one split the call is exactly attn_fwd and the array is not used.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)

attn_status_t attn_fwd_splitkv_noalloc(const attn_tensor_t* q, const attn_tensor_t* k,
                                       const attn_tensor_t* v, const attn_mask_t* bias_or_mask,
                                       int causal, float scale, int32_t num_splits,
                                       const attn_tensor_t* o, const attn_tensor_t* lse,
                                       void* stream);

/*
 * attn_fwd_varlen - the forward over packed variable-length sequences.
 *
 * A ragged batch is stored without padding: the rows of all sequences are
 * concatenated (the [total, heads, d] layout, token-major), and
 * cumulative offsets say where each sequence starts, so padding is never
 * computed ("flash-attention" (stanleyjacob.dev), Part II "Variable-length
 * batches: stop padding", and Lab 5; "FlashAttention, Explained", section
 * 14, document masking of packed batches). Sequence s attends its own
 * rows to its own keys only:
 *
 *     rows  [cu_seqlens_q[s], cu_seqlens_q[s+1])  of q, o, lse
 *     keys  [cu_seqlens_k[s], cu_seqlens_k[s+1])  of k, v
 *
 * with the same function per sequence as attn_fwd, including the
 * bottom-right causal alignment and the window of that sequence's lengths.
 *
 *   q    [1, H,  total_q, d]  bf16 or f32 (a [total_q, H, d] tensor is the
 *                             view with strides {., d, H*d, 1})
 *   k, v [1, Hk, total_k, d]  same dtype; Hk divides H
 *   cu_seqlens_q, cu_seqlens_k  DEVICE int32[num_seqs + 1], non-decreasing,
 *                             starting at 0 and ending at total_q / total_k.
 *                             Values outside [0, total] are clamped (the
 *                             kernels never leave the tensors), but then
 *                             the result is unspecified.
 *   num_seqs                  number of sequences (>= 0)
 *   max_seqlen_q              at least the longest query sequence (sizes
 *                             the grid; rows past it are not computed)
 *   window_mask               NULL, or an attn_mask_t with only the window
 *                             fields used (bias and kv_len must be NULL)
 *   causal, scale, stream     as for attn_fwd
 *   o    [1, H, total_q, d]   output, same dtype as q
 *   lse  [1, H, total_q, 1]   output, float32; stride[2] must be 1
 *
 * Rows of o / lse outside every sequence are not written. Layout,
 * alignment and error rules are those of attn_fwd.
 */
attn_status_t attn_fwd_varlen(const attn_tensor_t* q, const attn_tensor_t* k,
                              const attn_tensor_t* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                              const attn_mask_t* window_mask, int causal, float scale,
                              const attn_tensor_t* o, const attn_tensor_t* lse, void* stream);

/*
 * Backward pass (gradients of attn_fwd), recomputing the probabilities.
 *
 * Given the forward's inputs, its outputs O and LSE and the gradient dO of a
 * scalar loss with respect to O, computes
 *
 *     D_i = rowsum(dO_i o O_i),          P_ij = exp(S_ij - LSE_i),
 *     dV = P^T dO,   dP = dO V^T,       dS = P o (dP - D),
 *     dQ = scale * dS K,                 dK = scale * dS^T Q,
 *
 * with S, the masks and the window exactly as in attn_fwd; P is rebuilt
 * tile by tile from Q, K and LSE and never stored. ("Understanding
 * FlashAttention Pt 1", section 3.6; "FlashAttention, Explained", sections
 * 16-17; "FlashAttention: Mathematical Foundations...", section 4;
 * "flash-attention" (stanleyjacob.dev), Part VII.) With grouped K/V heads,
 * dK and dV of a K/V head sum over the query heads that read it. The bias,
 * when given, is treated as a constant (no gradient is returned for it).
 * The result is deterministic: no atomic accumulation is used.
 */

/* Bytes of workspace attn_bwd needs: 8 * B * H * Nq (two fp32 values per
   query row). -1 for a negative or too large extent. */
int64_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq);

/*
 * attn_bwd - enqueue the backward on `stream` (three kernels).
 *
 *   q, k, v, bias_or_mask, causal, scale   as passed to attn_fwd (bf16 only)
 *   o, lse     the outputs attn_fwd produced for them
 *   dout       [B, H, Nq, d] bf16, gradient with respect to o
 *   workspace  DEVICE pointer, 16-byte aligned, at least
 *              attn_bwd_workspace_size(B, H, Nq) bytes; scratch owned by the
 *              caller (contents on return undefined; concurrent calls need
 *              distinct workspaces)
 *   dq         [B, H, Nq, d] bf16 output
 *   dk, dv     [B, Hk, Nk, d] bf16 outputs
 *
 * Layout and alignment rules are those of attn_fwd for every tensor, and
 * the row stride of q and dout times 64 rows must also span less than
 * 2 GiB (ATTN_ERR_UNSUPPORTED otherwise); the outputs must not overlap the
 * inputs or each other. Keys no query sees get
 * dK = dV = 0 and a query row that sees no key gets dQ = 0. With B, H or Nq
 * equal to 0 no query sees any key: the call writes dK = dV = 0 (one small
 * kernel per tensor, when it has elements; their layout is checked as
 * above) and needs no workspace.
 */
attn_status_t attn_bwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                       const attn_tensor_t* o, const attn_tensor_t* lse,
                       const attn_tensor_t* dout, const attn_mask_t* bias_or_mask, int causal,
                       float scale, void* workspace, int64_t workspace_bytes,
                       const attn_tensor_t* dq, const attn_tensor_t* dk,
                       const attn_tensor_t* dv, void* stream);

/* Text describing the last non-OK status returned on the calling thread
   ("" if none). The pointer stays valid until the next call on this thread. */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_06_AMD_ATTN_H */
