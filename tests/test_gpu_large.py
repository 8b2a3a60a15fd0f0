"""Parity at sizes where one tensor holds more than 2^31 elements.

Every row and batch offset the kernels form is 64-bit; these cases place
rows past element 2^31 (byte 2^32) of the operands:

* forward and backward with B=2, H=4160, N=2048, d=128: each of q, k, v, o,
  dout, dq, dk and dv holds 2.18e9 elements. Three heads, the last among
  them, are compared with the oracle in full at the bars of the other
  parity tests.
* the split-key forward of one query against 2^24 + 1000 keys of one head
  (k and v hold 2.15e9 elements each). Every key row is zero except row
  j* near the end, so every score is exactly 0 except s* = scale q.k_j*,
  and the result has a closed form (the definition of softmax attention,
  evaluated in fp64 from the bf16 inputs):
      E = e^{s*} + (Nk - 1),  O = (e^{s*} v_j* + sum_{j != j*} v_j) / E,
      LSE = ln E.
  The plain (unsplit) forward is not run on this input: one lane pair
  would add 2^18 fp32 tile sums of identical size, whose rounding error
  is not bounded by the LSE bar; the split path adds ~1000 per split.
  [Understanding FlashAttention Pt 1, sections 2.1 and 3.4; flash-attention
  (stanleyjacob.dev), Part III, the split-key decoding path.]
"""

import math

import numpy as np
import pytest
import torch

import oracle
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import _banner, compare
from tests.test_gpu_bwd import _compare as compare_grads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield
    torch.cuda.empty_cache()


def _randn(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def test_many_heads_forward_and_backward():
    B, H, N, d = 2, 4160, 2048, 128
    assert B * H * N * d > 2 ** 31
    _banner(f"large: B={B} H={H} N={N} d={d} forward + backward")
    q, k, v, do = (_randn((B, H, N, d), 900 + i) for i in range(4))
    o, lse = ea.attn_fwd(q, k, v)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for b, h in ((0, 0), (1, 2077), (B - 1, H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1].double().cpu().numpy()
        ro, rl = oracle.attention_forward(sl(q), sl(k), sl(v), scale=scale)
        compare(sl(o), sl(lse), ro, rl, "bf16", f"large fwd head ({b}, {h})")
        ref = oracle.attention_backward(sl(q), sl(k), sl(v), sl(do), scale=scale)
        compare_grads([x[b:b + 1, h:h + 1].cpu() for x in (dq, dk, dv)], ref,
                      f"large bwd head ({b}, {h})")
    del dq, dk, dv
    # the causal forward of the same tensors (the persistent causal form:
    # 1040 heads per XCD, 260 rounds of tiles per workgroup, short tiles
    # back to back)
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    ea.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    for b, h in ((0, 0), (1, 2077), (B - 1, H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1].double().cpu().numpy()
        ro, rl = oracle.attention_forward(sl(q), sl(k), sl(v), scale=scale, causal=True)
        compare(sl(o), sl(lse), ro, rl, "bf16", f"large causal fwd head ({b}, {h})")
    del q, k, v, do, o, lse
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def spike_inputs():
    """One query, 2^24 + 1000 keys that are all zero except row j*, random
    values; with the fp64 sum of all value rows (computed on the CPU)."""
    d = 128
    nk = (1 << 24) + 1000
    assert nk * d > 2 ** 31
    js = nk - 37  # the one nonzero key row: byte offset past 2^32
    q = _randn((1, 1, 1, d), 910)
    v = _randn((1, 1, nk, d), 911)
    k = torch.zeros((1, 1, nk, d), device="cuda", dtype=torch.bfloat16)
    k[0, 0, js] = (1.4 * q[0, 0, 0].float()).to(torch.bfloat16)
    vsum = np.zeros(d)
    step = 1 << 20
    for a in range(0, nk, step):
        vsum += v[0, 0, a:a + step].cpu().to(torch.float64).sum(0).numpy()
    yield dict(q=q, k=k, v=v, js=js, nk=nk, d=d, vsum=vsum)
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_splits", [None, 1024])
def test_split_forward_beyond_2_31_key_elements(spike_inputs, num_splits):
    x = spike_inputs
    q, k, v, js, nk, d = x["q"], x["k"], x["v"], x["js"], x["nk"], x["d"]
    _banner(f"large: split forward, Nk={nk}, spike at key {js}, num_splits={num_splits}")
    o, lse = ea.attn_fwd_splitkv(q, k, v, num_splits=num_splits)
    torch.cuda.synchronize()

    scale = 1 / math.sqrt(d)
    s_star = scale * float(q[0, 0, 0].double().cpu().numpy() @ k[0, 0, js].double().cpu().numpy())
    vj = v[0, 0, js].double().cpu().numpy()
    # E and O relative to e^{s*} (s* ~ 16) to stay well inside fp64 range
    e_rel = 1.0 + (nk - 1) * math.exp(-s_star)
    ro = (vj + (x["vsum"] - vj) * math.exp(-s_star)) / e_rel
    rl = s_star + math.log(e_rel)
    compare(o[0, 0].double().cpu().numpy(), lse[0, 0].double().cpu().numpy(),
            ro[None], np.array([rl]), "bf16", f"large split Nk={nk} s*={s_star:.2f}")


def test_many_heads_biased_forward_d64():
    # the biased persistent form (d = 64, padded batches with a bias and key
    # lengths) on q, k, v, o of 2.18e9 elements each: rows of the last heads
    # lie past element 2^31; a bias shared by every batch and head
    B, H, N, d = 2, 8320, 2048, 64
    assert B * H * N * d > 2 ** 31
    _banner(f"large: B={B} H={H} N={N} d={d} biased forward with key lengths")
    q, k, v = (_randn((B, H, N, d), 950 + i) for i in range(3))
    g = torch.Generator(device="cuda")
    g.manual_seed(960)
    bias = 0.5 * torch.randn((1, 1, N, N), generator=g, device="cuda", dtype=torch.float32)
    kv_len = torch.tensor([1500, 2048], dtype=torch.int32, device="cuda")
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    ea.attn_fwd(q, k, v, bias=bias, kv_len=kv_len, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    scale = 1 / math.sqrt(d)
    bd = bias.double().cpu().numpy()
    kl = kv_len.cpu().numpy()
    for b, h in ((0, 0), (1, 4100), (B - 1, H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1].double().cpu().numpy()
        ro, rl = oracle.attention_forward(sl(q), sl(k), sl(v), scale=scale, bias=bd,
                                          kv_len=kl[b:b + 1])
        compare(sl(o), sl(lse), ro, rl, "bf16", f"large biased fwd head ({b}, {h})")
    del q, k, v, o, lse
