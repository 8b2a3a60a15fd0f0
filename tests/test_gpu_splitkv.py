"""Parity of the split-key forward (flash-decoding) with the fp64 CPU oracle.

attn_fwd_splitkv computes the same function as attn_fwd, so its expected
values are the oracle's ``attention_forward`` on the same seeded inputs, with
the same bars (bf16 O <= 2e-2, LSE <= 1e-3, -inf LSE and zero O rows for
fully masked rows). The cases cover split counts that do and do not divide
the key tiles, more splits requested than there are tiles, splits that are
empty for some rows (causal, per-batch key lengths), ragged tails, the bias,
grouped key/value heads, and the decoding workloads at full size (every
row, into NaN-filled outputs). [FlashAttention: Mathematical Foundations..., section 7, flash-decoding;
Understanding FlashAttention Pt 1, section 2.4, the merge of two blocks.]
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import (_banner, assert_all_written, compare, nan_outputs,
                                   run_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


def _cuda(x):
    return None if x is None else x.cuda()


def run_split(inp, num_splits=None, **kw):
    o, lse = ea.attn_fwd_splitkv(_cuda(inp["q"]), _cuda(inp["k"]), _cuda(inp["v"]),
                                 bias=_cuda(inp["bias"]), kv_len=_cuda(inp["kv_len"]),
                                 causal=inp["causal"], scale=inp["scale"],
                                 num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _inputs(B, H, Nq, Nk, d, causal=False, seed=0, Hk=None, bias=False, kv_len=None):
    w = workloads.Workload("split", B, H, Nq, Nk, d, causal=causal, seed=seed, Hk=Hk,
                           bias_std=0.5 if bias else None)
    inp = workloads.make_inputs(w)
    if kv_len is not None:
        inp["kv_len"] = torch.tensor(kv_len, dtype=torch.int32)
    return inp


def _oracle(inp):
    # grouped heads: query head h reads key/value head h // (H / Hk)
    rep = inp["q"].shape[1] // inp["k"].shape[1]
    if rep == 1:
        return run_oracle(inp)
    x = dict(inp)
    x["k"] = inp["k"].repeat_interleave(rep, dim=1)
    x["v"] = inp["v"].repeat_interleave(rep, dim=1)
    return run_oracle(x)


CASES = [
    # (B, H, Nq, Nk, d, causal, num_splits)
    (2, 3, 1, 1000, 128, False, 4),
    (2, 3, 1, 1000, 64, False, 7),       # 7 requested -> splits of 192 keys, 6 used
    (1, 4, 1, 65, 128, False, 2),        # second split holds one key
    (1, 2, 1, 4096, 128, False, 64),     # one tile per split
    (1, 2, 1, 700, 128, False, 1000),    # more splits requested than tiles
    (2, 2, 3, 1500, 128, True, 5),
    (2, 2, 128, 900, 128, True, 3),      # causal: early rows see no key of late splits
    (1, 2, 129, 1100, 64, True, 4),
    (1, 2, 300, 1300, 128, False, 3),    # more than one query tile per split
    (1, 1, 257, 257, 64, True, 2),
    (1, 2, 5, 3, 128, True, 2),          # a single tile: runs as the plain forward
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,ns", CASES)
def test_split_matches_oracle(B, H, Nq, Nk, d, causal, ns):
    _banner(f"split B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={ns}")
    inp = _inputs(B, H, Nq, Nk, d, causal=causal, seed=B * 1000 + Nk + ns)
    o, lse = run_split(inp, ns)
    ro, rl = _oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"split{ns}")


@pytest.mark.parametrize("d", [64, 128])
def test_split_bias_and_key_lengths(d):
    # batch entry 1 has no keys at all; entry 2 ends inside the first split
    inp = _inputs(3, 2, 2, 1200, d, bias=True, seed=21, kv_len=[1200, 0, 130])
    inp["bias"][..., 7] = -math.inf
    for causal in (False, True):
        inp["causal"] = causal
        _banner(f"split bias kv_len d={d} causal={causal}")
        o, lse = run_split(inp, 5)
        ro, rl = _oracle(inp)
        compare(o, lse, ro, rl, "bf16", f"split bias d={d} causal={causal}")
        assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("hk", [1, 4])
def test_split_grouped_kv_heads(hk):
    inp = _inputs(2, 8, 1, 2000, 128, Hk=hk, seed=22)
    _banner(f"split gqa Hk={hk}")
    o, lse = run_split(inp, 6)
    ro, rl = _oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"split gqa Hk={hk}")


# Packed heads (Nq <= 64, Hk < H): the H / Hk query heads of a key/value head
# share one row space of (H / Hk) * Nq rows. Row counts that leave a wave or
# a workgroup spanning two heads check the causal bounds; Nq = 65 is past
# the packing limit.
@pytest.mark.parametrize("H,Hk,Nq,d,causal,bias", [
    (8, 2, 5, 128, True, True),
    (8, 2, 33, 128, True, False),     # 132 rows: waves straddle heads
    (4, 1, 64, 64, True, False),      # 256 rows, 8-wave workgroups
    (16, 2, 3, 64, False, True),      # 24 rows
    (6, 3, 65, 128, True, False),     # not packed
])
def test_split_packed_heads(H, Hk, Nq, d, causal, bias):
    kv_len = [900, 333]
    inp = _inputs(2, H, Nq, 900, d, causal=causal, Hk=Hk, bias=bias, seed=27 + Nq,
                  kv_len=kv_len)
    _banner(f"split packed H={H} Hk={Hk} Nq={Nq} d={d} causal={causal} bias={bias}")
    o, lse = run_split(inp, 3)
    ro, rl = _oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"split packed H={H} Hk={Hk} Nq={Nq}")


def test_split_large_scores_move_reference():
    # scores near +-1e3, and each split's maximum differs widely: the merge
    # weights exp(LSE_s - M) span many orders of magnitude
    g = torch.Generator().manual_seed(23)
    q = (torch.randn(1, 2, 2, 64, generator=g) * 30).to(torch.bfloat16)
    k = (torch.randn(1, 2, 900, 64, generator=g) * 30).to(torch.bfloat16)
    v = torch.randn(1, 2, 900, 64, generator=g).to(torch.bfloat16)
    inp = {"q": q, "k": k, "v": v, "bias": None, "kv_len": None, "causal": False,
           "scale": 0.125}
    o, lse = run_split(inp, 5)
    ro, rl = run_oracle(inp)
    assert np.abs(rl).max() > 500
    compare(o, lse, ro, rl, "bf16", "split large scores")


def test_split_agrees_with_plain_forward_and_is_deterministic():
    inp = _inputs(2, 4, 7, 3000, 128, causal=True, seed=24)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o0, l0 = ea.attn_fwd(q, k, v, causal=True)
    o1, l1 = ea.attn_fwd_splitkv(q, k, v, causal=True, num_splits=6)
    o2, l2 = ea.attn_fwd_splitkv(q, k, v, causal=True, num_splits=6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # both round to bf16 once from fp32; they may differ by a rounding step
    assert (o0.float() - o1.float()).abs().max().item() <= 2e-2
    assert (l0 - l1).abs().max().item() <= 1e-3


def test_split_workspace_reused_across_calls():
    # one workspace, a larger call then a smaller one: stale partials of the
    # first call must not leak into the second
    ws = torch.empty(ea.splitkv_workspace_size(2, 4, 9, 128, 8), dtype=torch.uint8,
                     device="cuda")
    big = _inputs(2, 4, 9, 2500, 128, seed=25)
    small = _inputs(1, 2, 1, 900, 128, seed=26)
    for inp, ns in ((big, 8), (small, 3)):
        o, lse = run_split(inp, ns, workspace=ws)
        ro, rl = _oracle(inp)
        compare(o, lse, ro, rl, "bf16", f"workspace reuse splits={ns}")


def test_split_errors_raise():
    q = torch.randn(1, 1, 1, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 1, 1000, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(ea.AttnError, match="INVALID"):
        ea.attn_fwd_splitkv(q, k, k, num_splits=4,
                            workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ea.AttnError, match="UNSUPPORTED"):
        ea.attn_fwd_splitkv(q.float(), k.float(), k.float(), num_splits=4)


# --------------------------------------------------------------- decoding at full size

@pytest.mark.parametrize("name", sorted(workloads.DECODE))
def test_decode_full_size_every_row(name):
    # one query row per (batch, head): every one is compared with the oracle,
    # written into outputs pre-filled with NaN
    w = workloads.DECODE[name]
    _banner(f"decode full {name}")
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = nan_outputs(w.B, w.H, w.Nq, w.d, w.dtype)
    ea.attn_fwd_splitkv(q, k, v, scale=inp["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, name)
    assert torch.isfinite(lse_c).all()
    rep = w.H // w.kv_heads
    f = lambda t: t.double().numpy()
    go, gl, ro, rl = [], [], [], []
    for b in range(w.B):
        for h in range(w.H):
            hk = h // rep
            oo, ll = oracle.attention_forward(f(inp["q"][b:b + 1, h:h + 1]),
                                              f(inp["k"][b:b + 1, hk:hk + 1]),
                                              f(inp["v"][b:b + 1, hk:hk + 1]),
                                              scale=inp["scale"])
            ro.append(oo[0, 0])
            rl.append(ll[0, 0])
            go.append(o_c[b, h].double().numpy())
            gl.append(lse_c[b, h].double().numpy())
    compare(np.concatenate(go), np.concatenate(gl), np.concatenate(ro), np.concatenate(rl),
            "bf16", f"decode {name} every row")


def _random_split_cases(n, seed):
    """Seeded split-key problems: decoding-sized and larger query counts,
    grouped K/V heads (packed row spaces where Nq <= 64), causal or not, a
    bias and/or per-batch key lengths, split counts from 1 to 40."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(r.integers(1, 4))
        Hk = int(r.choice([1, 2, 3]))
        H = Hk * int(r.choice([1, 2, 4, 8]))
        Nq = int(r.choice([1, 2, 5, 17, 64, 65, 130]))
        Nk = int(r.integers(1, 3000))
        d = int(r.choice([64, 128]))
        causal = bool(r.integers(2))
        bias = bool(r.random() < 0.4)
        kv = [int(x) for x in r.integers(0, Nk + 50, B)] if r.random() < 0.5 else None
        ns = int(r.integers(1, 41))
        cases.append((B, H, Hk, Nq, Nk, d, causal, bias, kv, ns))
    return cases


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal,bias,kv,ns", _random_split_cases(10, 5151))
def test_split_random_problems(B, H, Hk, Nq, Nk, d, causal, bias, kv, ns):
    # seeded problems through the split-key forward and merge, compared in
    # full with the oracle [flash-attention, Part III; FlashAttention:
    # Mathematical Foundations..., section 7 (decoding)]
    _banner(f"split random B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d} causal={causal} "
            f"bias={bias} kv={kv} splits={ns}")
    inp = _inputs(B, H, Nq, Nk, d, causal=causal, Hk=Hk, bias=bias, kv_len=kv,
                  seed=31 * B + 7 * Nk + ns)
    o, lse = run_split(inp, ns)
    ro, rl = _oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"split random Nq={Nq} Nk={Nk} splits={ns}")
