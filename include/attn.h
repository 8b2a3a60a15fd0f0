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

#define ATTN_ABI_VERSION 1

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* malformed arguments: null pointer, shape mismatch, bad scale */
  ATTN_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels handle (head dim, dtype, stride, alignment) */
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

/* Optional additive terms on the scores. Both fields may be NULL. */
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
 *   scale                multiplies QK^T; must be finite and > 0 (callers
 *                        usually pass 1/sqrt(d))
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

/* Text describing the last non-OK status returned on the calling thread
   ("" if none). The pointer stays valid until the next call on this thread. */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_06_AMD_ATTN_H */
