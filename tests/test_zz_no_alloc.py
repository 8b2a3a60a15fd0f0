"""The entry point that allocates nothing, attn_fwd_splitkv_noalloc, against
attn_fwd_splitkv (same kernels, partials in a caller workspace) and the fp64
oracle.

Two calls in a row share the library's per-device scratch array, the second
with a smaller problem, so stale partials of the first call would show up in
the second. Each output must equal attn_fwd_splitkv's bit for bit (same
kernels, same split count) and meet the parity bars against the oracle
(bf16 O <= 2e-2, LSE <= 1e-3). A split count whose partials exceed the
scratch size is refused before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import _banner, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


def _inputs(B, H, Hk, Nq, Nk, d, seed, bias, kv_len):
    w = workloads.Workload("noalloc", B, H, Nq, Nk, d, seed=seed, Hk=Hk,
                           bias_std=0.5 if bias else None)
    inp = workloads.make_inputs(w)
    inp["kv_len"] = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    return inp


def _oracle(inp, causal):
    f = lambda t: None if t is None else t.double().numpy()
    k, v = inp["k"], inp["v"]
    rep = inp["q"].shape[1] // k.shape[1]
    if rep > 1:
        k, v = k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1)
    kv = None if inp["kv_len"] is None else inp["kv_len"].numpy()
    return oracle.attention_forward(f(inp["q"]), f(k), f(v), scale=inp["scale"],
                                    bias=f(inp["bias"]), kv_len=kv, causal=causal)


CALLS = [
    # (B, H, Hk, Nq, Nk, d, causal, bias, kv_len, num_splits): the first call
    # packs 4 query heads per key/value head and uses a bias and key
    # lengths; the second is smaller in every dimension
    (4, 8, 2, 3, 3000, 128, True, True, [3000, 1, 2047, 0], 6),
    (1, 2, 2, 1, 700, 64, False, False, None, 3),
]


def test_noalloc_matches_splitkv_two_calls():
    c = lambda t: None if t is None else t.cuda()
    for n, (B, H, Hk, Nq, Nk, d, causal, bias, kv_len, ns) in enumerate(CALLS):
        _banner(f"noalloc call {n}: B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d} "
                f"causal={causal} bias={bias} splits={ns}")
        inp = _inputs(B, H, Hk, Nq, Nk, d, seed=90 + n, bias=bias, kv_len=kv_len)
        q, k, v = c(inp["q"]), c(inp["k"]), c(inp["v"])
        args = dict(bias=c(inp["bias"]), kv_len=c(inp["kv_len"]), causal=causal,
                    scale=inp["scale"], num_splits=ns)
        o_ref, l_ref = ea.attn_fwd_splitkv(q, k, v, **args)
        o_na = torch.full_like(o_ref, float("nan"))
        l_na = torch.full_like(l_ref, float("nan"))
        ea.attn_fwd_splitkv_noalloc(q, k, v, out=o_na, lse=l_na, **args)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref), \
            f"call {n}: no-allocation output differs from attn_fwd_splitkv"
        ro, rl = _oracle(inp, causal)
        compare(o_na.double().cpu().numpy(), l_na.double().cpu().numpy(), ro, rl, "bf16",
                f"noalloc call {n}")
        if kv_len is not None and 0 in kv_len:
            b0 = kv_len.index(0)
            assert torch.all(o_na[b0] == 0) and torch.all(torch.isneginf(l_na[b0]))


def test_noalloc_refuses_partials_beyond_scratch():
    # 2 splits of 8 x 32 x 64 query rows at d = 128 need 16.9 MB of partials
    q = torch.zeros(8, 32, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(8, 32, 4096, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ea.AttnError, match="UNSUPPORTED.*scratch"):
        ea.attn_fwd_splitkv_noalloc(q, k, k, num_splits=2)
