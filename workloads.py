"""Seeded synthetic inputs for the attention forward.

This module only draws random numbers and names workloads. It holds none of
the attention arithmetic, and both sides of every comparison (the GPU library
and the CPU oracle) receive the very same tensors from it.

Recipe (fixed here, stated again in the design notes):

* ``torch.Generator().manual_seed(seed)`` on the CPU; draws in the order
  Q, K, V, then the extras (per-row Q factor, key lengths, bias).
* Every tensor is drawn as float32 ``randn``; any transform is applied in
  float32; then it is rounded once to the storage dtype (round to nearest
  even, which is what ``Tensor.to(torch.bfloat16)`` does).
* The bias, when present, is float32 with standard deviation ``bias_std``,
  shaped [1, H, Nq, Nk] so that it is shared by every batch entry.
* Key lengths are integers drawn uniformly from [kv_len_lo, kv_len_hi].
* Grouped key/value heads (``Hk`` set): K and V are drawn with Hk heads.
* Decoding workloads: one query row per (batch, head) against a long key
  sequence (the pages give no decode shape; these are typical serving ones:
  batch 8 at 16K keys, and one sequence at 64K keys, the length up to which
  the pages report near-constant decode latency).
* Sliding-window workloads: the long-context shape (B=1, H=16, N=16384,
  d=128) with a causal window of 4096 keys (a common local-attention size;
  the pages' example is 128 neighbouring tokens, too few tiles per row to
  measure anything but launch overhead).
* Packed variable-length batches (the pages' Lab 5: a ragged batch with
  lengths from a lognormal capped at 4096): the B sequence lengths are drawn
  first, n = clamp(round(exp(mu + sigma * z)), lo, cap) with z ~ N(0, 1),
  then Q, K, V packed token-major as [total, heads, d]; cu_seqlens are the
  cumulative lengths. Every sequence attends to itself (same lengths for
  queries and keys).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str = "bf16"            # "bf16" or "f32"
    causal: bool = False
    scale: Optional[float] = None  # None: 1/sqrt(d)
    value_scale: float = 1.0       # multiplies Q, K and V draws
    q_row_factor: Optional[tuple] = None   # (lo, hi): per-row U[lo, hi) factor on Q
    bias_std: Optional[float] = None        # dense bias [1, H, Nq, Nk] if set
    kv_len_range: Optional[tuple] = None    # (lo, hi) inclusive integer range
    seed: int = 0
    Hk: Optional[int] = None                # key/value heads (None: H)
    window: Optional[tuple] = None          # (left, right) sliding window
    varlen: Optional[tuple] = None          # (mu, sigma, lo, cap): packed lognormal lengths

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hk is None else self.Hk

    @property
    def softmax_scale(self) -> float:
        return (1.0 / math.sqrt(self.d)) if self.scale is None else float(self.scale)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def flops(self) -> float:
        """Nominal forward FLOPs, 4*B*H*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "H": self.H, "Nq": self.Nq,
            "Nk": self.Nk, "d": self.d, "dtype": self.dtype,
            "causal": self.causal, "scale": self.softmax_scale,
            "seed": self.seed, **({} if self.Hk is None else {"Hk": self.Hk}),
            **({} if self.window is None else {"window": list(self.window)}),
            **({} if self.varlen is None else {"lengths": "lognormal(mu=%g, sigma=%g) in [%d, %d]"
                                               % tuple(self.varlen), "sequences": self.B}),
        }

    def kv_bytes(self) -> int:
        """Bytes of K and V (each read once by a split-key forward)."""
        eb = 4 if self.dtype == "f32" else 2
        return 2 * self.B * self.kv_heads * self.Nk * self.d * eb


# The five workloads the method is measured on (seeds follow the config index).
CONFIGS = {
    "c1_f32_single_head": Workload("c1_f32_single_head", 1, 1, 256, 256, 64,
                                   dtype="f32", scale=1 / 8, seed=1),
    "c2_bf16_d64": Workload("c2_bf16_d64", 4, 16, 2048, 2048, 64,
                            scale=1 / 8, seed=2),
    "c2_bf16_d64_causal": Workload("c2_bf16_d64_causal", 4, 16, 2048, 2048, 64,
                                   scale=1 / 8, causal=True, seed=2),
    "c3_bf16_d128": Workload("c3_bf16_d128", 2, 32, 4096, 4096, 128, seed=3),
    "c3_bf16_d128_causal": Workload("c3_bf16_d128_causal", 2, 32, 4096, 4096,
                                    128, causal=True, seed=3),
    "c4_bf16_d128_long_causal": Workload("c4_bf16_d128_long_causal", 1, 16,
                                         16384, 16384, 128, causal=True,
                                         value_scale=0.5, q_row_factor=(1.0, 4.0),
                                         seed=4),
    "c5_bf16_d64_bias_padded": Workload("c5_bf16_d64_bias_padded", 8, 16, 1024,
                                        1024, 64, scale=1 / 8, bias_std=0.5,
                                        kv_len_range=(128, 1024), seed=5),
}

HEADLINE = "c3_bf16_d128"

# Decoding (one query row per head) for the split-key forward.
DECODE = {
    "decode_b8_h32_k16k_d128": Workload("decode_b8_h32_k16k_d128", 8, 32, 1, 16384, 128,
                                        seed=6),
    "decode_gqa_b8_h32_hk8_k16k_d128": Workload("decode_gqa_b8_h32_hk8_k16k_d128", 8, 32, 1,
                                                16384, 128, Hk=8, seed=6),
    "decode_b1_h32_k64k_d128": Workload("decode_b1_h32_k64k_d128", 1, 32, 1, 65536, 128,
                                        seed=7),
}

# Sliding-window (local) attention.
WINDOW = {
    "local_b1_h16_n16k_w4096_d128": Workload("local_b1_h16_n16k_w4096_d128", 1, 16, 16384,
                                             16384, 128, causal=True, window=(4096, 0),
                                             seed=8),
}

# Packed variable-length sequences (Nq = Nk = the length cap).
VARLEN = {
    "varlen_s16_h16_d128_lognormal_causal": Workload(
        "varlen_s16_h16_d128_lognormal_causal", 16, 16, 4096, 4096, 128, causal=True,
        varlen=(math.log(1024.0), 0.8, 32, 4096), seed=9),
}

ALL = {**CONFIGS, **DECODE, **WINDOW, **VARLEN}


def _storage(dtype: str):
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict with q, k, v (storage dtype, [B, H, N, d], contiguous),
    bias (float32 [1, H, Nq, Nk] or None), kv_len (int32 [B] or None),
    causal, scale (the float32-representable softmax scale as a Python float).
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else int(seed))
    st = _storage(w.dtype)
    q = torch.randn((w.B, w.H, w.Nq, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.kv_heads, w.Nk, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.kv_heads, w.Nk, w.d), generator=g, dtype=torch.float32)
    if w.value_scale != 1.0:
        q.mul_(w.value_scale)
        k.mul_(w.value_scale)
        v.mul_(w.value_scale)
    if w.q_row_factor is not None:
        lo, hi = w.q_row_factor
        f = torch.rand((w.B, w.H, w.Nq, 1), generator=g, dtype=torch.float32)
        q.mul_(lo + (hi - lo) * f)
    kv_len = None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        kv_len = torch.randint(int(lo), int(hi) + 1, (w.B,), generator=g,
                               dtype=torch.int64).to(torch.int32)
    bias = None
    if w.bias_std is not None:
        bias = torch.randn((1, w.H, w.Nq, w.Nk), generator=g,
                           dtype=torch.float32) * float(w.bias_std)
    scale32 = float(torch.tensor(w.softmax_scale, dtype=torch.float32))
    return {
        "q": q.to(st).contiguous(), "k": k.to(st).contiguous(),
        "v": v.to(st).contiguous(), "bias": bias, "kv_len": kv_len,
        "causal": bool(w.causal), "scale": scale32,
    }


def make_varlen_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw a packed variable-length batch for workload ``w`` (w.varlen set).

    Returns q [T, H, d], k, v [T, Hk, d] (storage dtype, contiguous), lens
    (int64 [B]), cu (int32 [B + 1] cumulative lengths), max_len, causal,
    scale.
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else int(seed))
    mu, sigma, lo, cap = w.varlen
    z = torch.randn((w.B,), generator=g, dtype=torch.float32)
    lens = torch.exp(mu + sigma * z).round().clamp(lo, cap).to(torch.int64)
    T = int(lens.sum())
    st = _storage(w.dtype)
    q = torch.randn((T, w.H, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((T, w.kv_heads, w.d), generator=g, dtype=torch.float32)
    v = torch.randn((T, w.kv_heads, w.d), generator=g, dtype=torch.float32)
    cu = torch.zeros(w.B + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lens, 0)
    scale32 = float(torch.tensor(w.softmax_scale, dtype=torch.float32))
    return {"q": q.to(st).contiguous(), "k": k.to(st).contiguous(), "v": v.to(st).contiguous(),
            "lens": lens, "cu": cu.to(torch.int32), "max_len": int(lens.max()),
            "causal": bool(w.causal), "scale": scale32}


def small(name: str, **overrides) -> Workload:
    """A reduced copy of a named workload (same dtype, masks and value
    distribution) for checks the oracle can evaluate in full."""
    return ALL[name].with_(**overrides)
