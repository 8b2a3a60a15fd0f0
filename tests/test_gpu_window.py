"""Parity of the sliding-window (local attention) forward with the oracle.

Key j takes part for query i only if i + (Nk - Nq) - left <= j <= i +
(Nk - Nq) + right (a negative bound leaves that side open; causal sets
right = 0). Expected values are the oracle's ``attention_forward`` with the
same window on the same seeded inputs, at the bars of the other parity
tests. The cases cover bands narrower than a tile, bands of several tiles
(the workgroup skips whole tiles before its first row's band), one-sided
windows, unequal query and key counts (rows with no key at all), the bias,
key lengths, both dtypes, the split-key path and packed grouped heads.
[Understanding FlashAttention Pt 1, section 3.5; FlashAttention, Explained,
section 14; flash-attention, Part III, window_size.]
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import (_banner, assert_all_written, compare, compare_rows,
                                   full_size_rows, nan_outputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


def _cuda(x):
    return None if x is None else x.cuda()


def _inputs(B, H, Nq, Nk, d, dtype="bf16", seed=0, Hk=None, bias=False, kv_len=None):
    w = workloads.Workload("window", B, H, Nq, Nk, d, dtype=dtype, seed=seed, Hk=Hk,
                           bias_std=0.5 if bias else None)
    inp = workloads.make_inputs(w)
    if kv_len is not None:
        inp["kv_len"] = torch.tensor(kv_len, dtype=torch.int32)
    return inp


def _oracle(inp, causal, window):
    f = lambda t: None if t is None else t.double().numpy()
    k, v = inp["k"], inp["v"]
    rep = inp["q"].shape[1] // k.shape[1]
    if rep > 1:
        k, v = k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1)
    kv = None if inp["kv_len"] is None else inp["kv_len"].numpy()
    return oracle.attention_forward(f(inp["q"]), f(k), f(v), scale=inp["scale"],
                                    bias=f(inp["bias"]), kv_len=kv, causal=causal,
                                    window=window)


def _gpu_run(inp, causal, window, split=False, num_splits=None):
    args = dict(bias=_cuda(inp["bias"]), kv_len=_cuda(inp["kv_len"]), causal=causal,
                scale=inp["scale"], window=window)
    q, k, v = _cuda(inp["q"]), _cuda(inp["k"]), _cuda(inp["v"])
    if split:
        o, lse = ea.attn_fwd_splitkv(q, k, v, num_splits=num_splits, **args)
    else:
        o, lse = ea.attn_fwd(q, k, v, **args)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


CASES = [
    # (Nq, Nk, d, dtype, causal, window)
    (300, 300, 128, "bf16", True, (128, 0)),     # 128 neighbouring keys
    (300, 300, 64, "bf16", False, (100, 30)),
    (257, 257, 128, "bf16", False, (0, 0)),      # the diagonal key only
    (200, 333, 64, "bf16", False, (-1, 50)),     # right bound only
    (333, 200, 128, "bf16", False, (70, -1)),    # left bound only; early rows see nothing
    (500, 500, 128, "bf16", True, (64, -1)),
    (700, 700, 64, "bf16", True, (200, 5)),      # causal overrides the right bound
    (2000, 2000, 128, "bf16", True, (300, 0)),   # workgroups skip tiles before the band
    (2000, 2000, 64, "bf16", False, (450, 450)),
    (130, 130, 64, "f32", False, (20, 10)),
    (130, 150, 128, "f32", True, (33, -1)),
    (400, 400, 64, "f32", True, (100, 0)),
]


@pytest.mark.parametrize("Nq,Nk,d,dtype,causal,window", CASES)
def test_window_matches_oracle(Nq, Nk, d, dtype, causal, window):
    _banner(f"window Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} window={window}")
    inp = _inputs(1, 2, Nq, Nk, d, dtype=dtype, seed=Nq + Nk + d)
    o, lse = _gpu_run(inp, causal, window)
    ro, rl = _oracle(inp, causal, window)
    compare(o, lse, ro, rl, dtype, f"window {window}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_with_bias_and_key_lengths(dtype):
    inp = _inputs(3, 2, 260, 300, 64, dtype=dtype, bias=True, seed=41, kv_len=[300, 0, 170])
    inp["bias"][..., 11] = -math.inf
    for causal, window in ((True, (90, 0)), (False, (40, 70))):
        _banner(f"window bias kv_len {dtype} causal={causal} window={window}")
        o, lse = _gpu_run(inp, causal, window)
        ro, rl = _oracle(inp, causal, window)
        compare(o, lse, ro, rl, dtype, f"window bias {window}")
        assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("Nq,Hk,window,ns", [
    (1, None, (1000, 0), 4),      # decoding against the last 1001 keys
    (1, 2, (700, -1), 5),         # packed heads
    (40, 2, (300, 0), 3),
    (300, None, (500, 20), 4),
])
def test_window_split(Nq, Hk, window, ns):
    _banner(f"window split Nq={Nq} Hk={Hk} window={window} splits={ns}")
    inp = _inputs(2, 4, Nq, 3000, 128, seed=42 + Nq, Hk=Hk)
    causal = window[1] == 0
    o, lse = _gpu_run(inp, causal, window, split=True, num_splits=ns)
    ro, rl = _oracle(inp, causal, window)
    compare(o, lse, ro, rl, "bf16", f"window split {window}")


def test_window_equivalences():
    # an open window is the plain forward and (left open, right 0) is the
    # causal one: bit-identical launches
    inp = _inputs(1, 2, 333, 333, 128, seed=43)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o0, l0 = ea.attn_fwd(q, k, v)
    o1, l1 = ea.attn_fwd(q, k, v, window=(-1, -1))
    oc, lc = ea.attn_fwd(q, k, v, causal=True)
    o2, l2 = ea.attn_fwd(q, k, v, window=(None, 0))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(oc, o2) and torch.equal(lc, l2)


@pytest.mark.parametrize("name", sorted(workloads.WINDOW))
def test_window_full_size_every_tile(name):
    # NaN-filled outputs; one row of every 128-row query tile and every row
    # of the first and last head against the oracle
    w = workloads.WINDOW[name]
    _banner(f"window full {name}")
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o, lse = nan_outputs(w.B, w.H, w.Nq, w.d, w.dtype)
    ea.attn_fwd(q, k, v, causal=w.causal, scale=inp["scale"], window=w.window, out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, name)
    assert torch.isfinite(lse_c).all()
    f = lambda t: t.double().numpy()
    qd, kd, vd = f(inp["q"]), f(inp["k"]), f(inp["v"])

    def oracle_rows(part):
        return oracle.attention_rows(qd, kd, vd, part, scale=inp["scale"], causal=w.causal,
                                     window=w.window)

    compare_rows(o_c, lse_c, full_size_rows(w), oracle_rows, w.dtype, f"window full {name}")


def _random_window_cases(n, seed):
    """Seeded windowed problems through the per-tile and split kernels: both
    dtypes and head dimensions, grouped heads, one- and two-sided bands of
    every width (0 to past the keys), causal or not, a bias and key lengths."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        dtype = "f32" if r.random() < 0.25 else "bf16"
        d = int(r.choice([64, 128]))
        B = int(r.integers(1, 3))
        Hk = int(r.choice([1, 2]))
        H = Hk * int(r.choice([1, 2]))
        Nq = int(r.integers(1, 900))
        Nk = int(r.integers(1, 900))
        causal = bool(r.integers(2))
        window = (int(r.integers(-1, 700)), int(r.integers(-1, 300)))
        bias = bool(r.random() < 0.3)
        kv = [int(x) for x in r.integers(0, Nk + 30, B)] if r.random() < 0.4 else None
        split = dtype == "bf16" and r.random() < 0.3
        cases.append((dtype, d, B, H, Hk, Nq, Nk, causal, window, bias, kv, split))
    return cases


@pytest.mark.parametrize("dtype,d,B,H,Hk,Nq,Nk,causal,window,bias,kv,split",
                         _random_window_cases(10, 8484))
def test_window_random_problems(dtype, d, B, H, Hk, Nq, Nk, causal, window, bias, kv, split):
    # seeded windowed problems, every row compared with the oracle (reading
    # of the band: around the bottom-right diagonal, a negative bound open)
    # [flash-attention, Part III, window_size; FlashAttention, Explained,
    # section 14]
    _banner(f"window random {dtype} d={d} B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} causal={causal} "
            f"window={window} bias={bias} kv={kv} split={split}")
    inp = _inputs(B, H, Nq, Nk, d, dtype=dtype, seed=11 * Nq + Nk + d, Hk=Hk, bias=bias,
                  kv_len=kv)
    o, lse = _gpu_run(inp, causal, window, split=split, num_splits=3 if split else None)
    ro, rl = _oracle(inp, causal, window)
    compare(o, lse, ro, rl, dtype, f"window random {window}")
