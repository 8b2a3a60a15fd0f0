// Internal parameter block handed from the C ABI front end to the kernel
// launchers. Plain data: every pointer is a device pointer, strides are in
// elements and already validated (non-negative, alignment checked).
#pragma once

#include <stdint.h>

namespace attn {

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
  float scale_log2;          // scale * log2(e): scores go to base-2 units
};

// How the flat workgroup index maps onto (batch, head, query tile).
struct TileMap {
  int32_t n_qtiles;      // ceil(Nq / tile rows)
  int32_t total;         // B * H * n_qtiles
  int32_t per_xcd;       // ceil(total / 8)
  int32_t batch_inner;   // 1: batch index varies fastest (shared bias reuse)
  int32_t reverse_q;     // 1: longest query tiles first (causal)
};

// Host-side launchers (one per kernel family). Return a hipError_t value.
int launch_fwd_bf16(const FwdParams& p, int d, void* stream);
int launch_fwd_f32(const FwdParams& p, int d, void* stream);

}  // namespace attn
