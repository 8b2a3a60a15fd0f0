"""Parity of the HIP backward (through the C ABI) with the fp64 oracle.

The GPU forward produces O and LSE; the GPU backward then gets the same
seeded dO, and its dQ, dK, dV are compared with ``oracle.attention_backward``
(which rebuilds P from Q, K itself, in fp64). Bar, per gradient tensor X:

    max |X_gpu - X_oracle| <= TOL_GRAD * max |X_oracle|

TOL_GRAD = 2e-2. Where it comes from: the kernels multiply bf16 operands
(P and dS are rounded to bf16 before the dV, dK and dQ products, as the
pages' fast kernels do, relative error 2^-9 per element), accumulate in
fp32 and round the result to bf16 once (2^-9 of |X|); over n terms of mixed
sign the rounding errors add like sqrt(n), so for the sizes here the
expected error is a few 2^-9 of the largest entry. The printed figures show
the margin case by case. Also: NaN-free, rows that see no key have dQ = 0,
keys no query sees have dK = dV = 0, and repeated calls are bitwise equal.
[Understanding FlashAttention Pt 1, section 3.6; FlashAttention, Explained,
sections 16-17; flash-attention, Part VII.]
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import _banner

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


def _case(B, H, Hk, Nq, Nk, d, seed, bias=False):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hk, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hk, Nk, d, generator=g).to(torch.bfloat16)
    do = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    bb = (torch.randn(1, H, Nq, Nk, generator=g) * 0.5) if bias else None
    return q, k, v, do, bb


def _gpu_grads(q, k, v, do, bias=None, kv_len=None, causal=False, window=None, scale=None):
    c = lambda t: None if t is None else t.cuda()
    qg, kg, vg, dog = c(q), c(k), c(v), c(do)
    o, lse = ea.attn_fwd(qg, kg, vg, bias=c(bias), kv_len=c(kv_len), causal=causal,
                         scale=scale, window=window)
    dq, dk, dv = ea.attn_bwd(qg, kg, vg, o, lse, dog, bias=c(bias), kv_len=c(kv_len),
                             causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    return dq, dk, dv


def _compare(got, ref, what):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().cpu().numpy()
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        scale = max(np.abs(r).max(), 1e-12)
        e = np.abs(g - r).max() / scale
        errs.append(f"{name} {e:.2e}")
        assert e <= TOL_GRAD, f"{what}: {name} relative error {e}"
    _banner(f"{what}: max|err|/max|ref| " + ", ".join(errs))


def _check(B, H, Hk, Nq, Nk, d, seed, causal=False, window=None, bias=False, kv_len=None):
    q, k, v, do, bb = _case(B, H, Hk, Nq, Nk, d, seed, bias)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    got = _gpu_grads(q, k, v, do, bb, kl, causal, window)
    f = lambda t: None if t is None else t.double().numpy()
    ref = oracle.attention_backward(f(q), f(k), f(v), f(do), scale=1 / math.sqrt(d),
                                    bias=f(bb), kv_len=kv_len, causal=causal, window=window)
    _compare(got, ref, f"bwd B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d} causal={causal} "
                       f"window={window} bias={bias} kv_len={kv_len}")
    return got, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(128, 128), (300, 300), (200, 333), (65, 190), (1, 77)])
def test_bwd_matches_oracle(d, causal, nq, nk):
    _check(1, 2, 2, nq, nk, d, seed=nq + nk + d, causal=causal)


def test_bwd_rows_without_keys_and_unseen_keys():
    # causal with Nq > Nk: the first Nq - Nk rows see no key (dQ = 0); key
    # lengths leave keys no query sees (dK = dV = 0)
    got, ref = _check(2, 2, 2, 190, 70, 64, seed=81, causal=True)
    assert torch.all(got[0][:, :, :120].cpu() == 0)
    got, _ = _check(2, 2, 2, 150, 300, 128, seed=82, kv_len=[300, 100])
    assert torch.all(got[1][1, :, 100:].cpu() == 0) and torch.all(got[2][1, :, 100:].cpu() == 0)


@pytest.mark.parametrize("q_shape,kv_shape", [((2, 4, 0, 128), (2, 2, 300, 128)),
                                               ((2, 0, 10, 64), (2, 2, 77, 64))])
def test_bwd_empty_query_side_zeroes_dk_dv(q_shape, kv_shape):
    # no query rows (or no query heads) but keys present: no query sees any
    # key, so dK = dV = 0; the outputs start as NaN and dv is a strided view
    _banner(f"bwd empty query side q={q_shape} kv={kv_shape}")
    q = torch.zeros(q_shape, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(kv_shape, device="cuda").to(torch.bfloat16)
    v = torch.randn(kv_shape, device="cuda").to(torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros(q_shape[:3], dtype=torch.float32, device="cuda")
    dk = torch.full(kv_shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    B, Hk, Nk, d = kv_shape
    dv_store = torch.full((B, Nk, Hk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = dv_store.transpose(1, 2)
    _, dk2, dv2 = ea.attn_bwd(q, k, v, o, lse, torch.zeros_like(q), dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk.cpu() == 0) and torch.all(dv_store.cpu() == 0)


@pytest.mark.parametrize("hk", [1, 2])
def test_bwd_grouped_heads(hk):
    _check(2, 4, hk, 260, 260, 128, seed=83, causal=True)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_bias_and_key_lengths(d):
    _check(2, 2, 2, 170, 230, d, seed=84, bias=True, kv_len=[230, 57])


@pytest.mark.parametrize("window,causal", [((100, 0), True), ((40, 70), False), ((-1, 30), False)])
def test_bwd_window(window, causal):
    _check(1, 2, 2, 400, 400, 128, seed=85, causal=causal, window=window)


def test_bwd_deterministic():
    q, k, v, do, _ = _case(1, 4, 2, 333, 500, 128, seed=86)
    a = _gpu_grads(q, k, v, do, causal=True)
    b = _gpu_grads(q, k, v, do, causal=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_heads():
    # the headline shape (B=2, H=32, N=4096, d=128) computed in full on the
    # GPU; two heads are checked against the oracle in full
    w = workloads.CONFIGS["c3_bf16_d128"]
    inp = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(87)
    do = torch.randn(w.B, w.H, w.Nq, w.d, generator=g).to(torch.bfloat16)
    got = _gpu_grads(inp["q"], inp["k"], inp["v"], do, scale=inp["scale"])
    for b, h in ((0, 0), (1, 31)):
        sl = lambda t: t[b:b + 1, h:h + 1].double().numpy()
        ref = oracle.attention_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(do),
                                        scale=inp["scale"])
        _compare([x[b:b + 1, h:h + 1] for x in got], ref, f"bwd full c3 head ({b}, {h})")


def _random_bwd_cases(n, seed):
    """Seeded backward problems: ragged query and key counts, grouped K/V
    heads, causal, a window or neither, a bias and/or per-batch key lengths."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(r.integers(1, 3))
        Hk = int(r.choice([1, 2]))
        H = Hk * int(r.choice([1, 2, 3]))
        Nq = int(r.integers(1, 400))
        Nk = int(r.integers(1, 400))
        d = int(r.choice([64, 128]))
        mode = int(r.integers(3))
        causal = mode == 1
        window = (int(r.integers(0, 200)), int(r.integers(-1, 100))) if mode == 2 else None
        bias = bool(r.random() < 0.3)
        kv = [int(x) for x in r.integers(0, Nk + 20, B)] if r.random() < 0.4 else None
        cases.append((B, H, Hk, Nq, Nk, d, causal, window, bias, kv))
    return cases


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal,window,bias,kv", _random_bwd_cases(10, 6161))
def test_bwd_random_problems(B, H, Hk, Nq, Nk, d, causal, window, bias, kv):
    # seeded problems, dQ, dK, dV against the oracle at the gradient bar
    # [FlashAttention, Explained, section 17; flash-attention, Part VII]
    _check(B, H, Hk, Nq, Nk, d, seed=13 * Nq + Nk + d, causal=causal, window=window, bias=bias,
           kv_len=kv)
