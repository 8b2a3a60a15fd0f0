"""Parity of the HIP forward (through the C ABI) with the fp64 CPU oracle.

Both sides read the same seeded bytes (bf16 or f32, widened exactly to fp64
for the oracle). Bars, written here and nowhere else:
  * max |O_gpu - O_oracle| <= 2e-2 for bf16 O, <= 1e-5 for f32 O;
  * max |LSE_gpu - LSE_oracle| <= 1e-3;
  * no NaN anywhere; a -inf LSE (fully masked row) must match exactly and
    its O row must be exactly zero.
Small cases are compared element by element; the five full-size workloads
are run in the launch configuration the benchmark times, into outputs
pre-filled with NaN, and checked on one row of every query tile, on every
row of the first and last head, and on properties that hold at any size.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

pytestmark = pytest.mark.gpu

TOL_O = {"bf16": 2e-2, "f32": 1e-5}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


def _banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _to_gpu(x):
    return None if x is None else x.cuda()


def run_gpu(inp, **kw):
    o, lse = ea.attn_fwd(_to_gpu(inp["q"]), _to_gpu(inp["k"]), _to_gpu(inp["v"]),
                         bias=_to_gpu(inp["bias"]), kv_len=_to_gpu(inp["kv_len"]),
                         causal=inp["causal"], scale=inp["scale"], **kw)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def run_oracle(inp):
    f = lambda t: None if t is None else t.double().numpy()
    kv = None if inp["kv_len"] is None else inp["kv_len"].numpy()
    return oracle.attention_forward(f(inp["q"]), f(inp["k"]), f(inp["v"]),
                                    scale=inp["scale"], bias=f(inp["bias"]),
                                    kv_len=kv, causal=inp["causal"])


def compare(o, lse, ro, rl, dtype, what=""):
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), f"{what}: -inf LSE pattern differs"
    if dead.any():
        assert np.all(o[dead] == 0.0), f"{what}: fully masked rows must be zero"
    err_o = np.abs(o - ro).max() if o.size else 0.0
    live = ~dead
    err_l = np.abs(lse[live] - rl[live]).max() if live.any() else 0.0
    # reported, not asserted: the mean error, and the floor set by rounding
    # the oracle's own O to the output dtype
    mean_o = np.abs(o - ro).mean() if o.size else 0.0
    rdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    floor_o = (np.abs(torch.from_numpy(ro).to(rdt).double().numpy() - ro).max() if o.size else 0.0)
    _banner(f"{what}: max|dO|={err_o:.3e} mean|dO|={mean_o:.3e} (rounding floor {floor_o:.3e}) "
            f"max|dLSE|={err_l:.3e}")
    assert err_o <= TOL_O[dtype], f"{what}: O error {err_o}"
    assert err_l <= TOL_LSE, f"{what}: LSE error {err_l}"


def check(w: workloads.Workload, seed=None):
    _banner(f"{w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} "
            f"causal={w.causal} seed={seed}")
    inp = workloads.make_inputs(w, seed=seed)
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    compare(o, lse, ro, rl, w.dtype, w.name)
    return inp, o, lse


# --------------------------------------------------------------- reduced workloads

def test_config1_full_size_f32():
    w = workloads.CONFIGS["c1_f32_single_head"]
    check(w)
    check(w, seed=101)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [333, 512])
def test_config2_reduced(causal, n):
    w = workloads.small("c2_bf16_d64", B=2, H=3, Nq=n, Nk=n, causal=causal)
    check(w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [300, 640])
def test_config3_reduced(causal, n):
    w = workloads.small("c3_bf16_d128", B=2, H=2, Nq=n, Nk=n, causal=causal)
    check(w)


def test_config4_reduced():
    w = workloads.small("c4_bf16_d128_long_causal", H=2, Nq=1000, Nk=1000)
    check(w)
    check(w, seed=104)


@pytest.mark.parametrize("n", [300, 1024])
def test_config5_reduced(n):
    w = workloads.small("c5_bf16_d64_bias_padded", B=4, H=2, Nq=n, Nk=n,
                        kv_len_range=(1, n))
    check(w)


# --------------------------------------------------------------- edge cases

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 200), (70, 1), (129, 65), (65, 190), (200, 77)])
def test_unequal_and_tiny_lengths(d, dtype, causal, nq, nk):
    # causal with Nq > Nk leaves the first Nq - Nk rows fully masked
    w = workloads.Workload("edge", 1, 2, nq, nk, d, dtype=dtype, causal=causal, seed=7)
    check(w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bias_broadcast_and_key_lengths(dtype):
    g = torch.Generator().manual_seed(11)
    B, H, Nq, Nk, d = 3, 4, 150, 170, 64
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, H, Nq, d, generator=g).to(st)
    k = torch.randn(B, H, Nk, d, generator=g).to(st)
    v = torch.randn(B, H, Nk, d, generator=g).to(st)
    kv_len = torch.tensor([170, 0, 64], dtype=torch.int32)
    for bshape in [(B, 1, Nq, Nk), (1, H, Nq, Nk), (B, H, Nq, Nk), (1, 1, Nq, Nk)]:
        bias = torch.randn(*bshape, generator=g) * 2.0
        bias[..., 5] = -math.inf      # a masked key through the bias
        for causal in (False, True):
            inp = {"q": q, "k": k, "v": v, "bias": bias, "kv_len": kv_len,
                   "causal": causal, "scale": 0.125}
            o, lse = run_gpu(inp)
            ro, rl = run_oracle(inp)
            compare(o, lse, ro, rl, dtype, f"bias{bshape} causal={causal}")
            assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_key_lengths_without_bias(d, dtype, causal):
    # key lengths alone (no bias tensor): no keys, one key, exactly one and
    # just over one 64-key tile, a ragged tail and all keys; the unbiased,
    # unmasked bf16 kernel computes half of each tile's probabilities ahead
    # of the tile, so partial and empty tiles pass through that path too
    g = torch.Generator().manual_seed(18)
    B, H, Nq, Nk = 6, 2, 150, 300
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, H, Nq, d, generator=g).to(st)
    k = torch.randn(B, H, Nk, d, generator=g).to(st)
    v = torch.randn(B, H, Nk, d, generator=g).to(st)
    kv_len = torch.tensor([Nk, 0, 1, 64, 65, 190], dtype=torch.int32)
    inp = {"q": q, "k": k, "v": v, "bias": None, "kv_len": kv_len, "causal": causal,
           "scale": d ** -0.5}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    compare(o, lse, ro, rl, dtype, f"key lengths d={d} causal={causal}")
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("aligned", [True, False])
def test_bias_tiles_staged_and_direct(causal, aligned):
    # d = 64 with a bias whose rows start 16-byte aligned and a key count
    # divisible by 4: bias tiles go through LDS (the last, ragged tile with
    # clamped chunks); a bias view shifted by one element takes the direct
    # loads instead. Same inputs, same oracle, both within the bars.
    g = torch.Generator().manual_seed(20)
    B, H, Nq, Nk, d = 3, 2, 200, 324, 64
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    # rows 4 floats apart from one another (16-byte multiples), the view on
    # the device so that its strides and offset reach the library as they are
    store = (torch.randn(B, H, Nq, Nk + 4, generator=g) * 0.7).cuda()
    bias = store[..., :Nk] if aligned else store[..., 1:Nk + 1]
    kv_len = torch.tensor([Nk, 5, 130], dtype=torch.int32)
    inp = {"q": q, "k": k, "v": v, "bias": bias, "kv_len": kv_len, "causal": causal,
           "scale": 0.125}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle({**inp, "bias": bias.cpu()})
    compare(o, lse, ro, rl, "bf16", f"bias tiles aligned={aligned} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_many_tiles_per_wave(d, causal):
    # fp32 with 1000 keys: every wave of a workgroup runs several key tiles
    # before the merge (and, causal, the waves of early rows run fewer or
    # none); key lengths cut some batches short, one to nothing.
    g = torch.Generator().manual_seed(22)
    B, H, Nq, Nk = 3, 2, 90, 1000
    q = torch.randn(B, H, Nq, d, generator=g) * 1.5
    k = torch.randn(B, H, Nk, d, generator=g)
    v = torch.randn(B, H, Nk, d, generator=g)
    kv_len = torch.tensor([Nk, 617, 0], dtype=torch.int32)
    inp = {"q": q, "k": k, "v": v, "bias": None, "kv_len": kv_len, "causal": causal,
           "scale": d ** -0.5}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    compare(o, lse, ro, rl, "f32", f"f32 many tiles d={d} causal={causal}")
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse[2]))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("aligned", [True, False])
def test_f32_bias_vector_and_scalar_loads(d, causal, aligned):
    # fp32: with 16-byte aligned bias rows a lane's four bias values arrive
    # as one vector load, except where the four keys run past Nk (Nk = 301:
    # the last group falls back to single loads); a view shifted by one
    # element takes single loads throughout. Several 16-row workgroups, key
    # tiles spread over the waves of each, a ragged last tile.
    g = torch.Generator().manual_seed(21)
    B, H, Nq, Nk = 2, 2, 70, 301
    q = torch.randn(B, H, Nq, d, generator=g)
    k = torch.randn(B, H, Nk, d, generator=g)
    v = torch.randn(B, H, Nk, d, generator=g)
    store = (torch.randn(B, H, Nq, Nk + 3, generator=g) * 0.7).cuda()
    bias = store[..., :Nk] if aligned else store[..., 1:Nk + 1]
    kv_len = torch.tensor([Nk, 150], dtype=torch.int32)
    inp = {"q": q, "k": k, "v": v, "bias": bias, "kv_len": kv_len, "causal": causal,
           "scale": d ** -0.5}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle({**inp, "bias": bias.cpu()})
    compare(o, lse, ro, rl, "f32", f"f32 bias d={d} aligned={aligned} causal={causal}")


@pytest.mark.parametrize("B,lens", [
    (7, [300, 64, 300, 0, 1, 129, 64]),        # odd count (the middle rank runs alone), ties
    (64, None),                                # the most batches ranked on the device
    (65, None),                                # one more: the unpaired order
])
def test_bias_key_lengths_paired_batches(B, lens):
    # d = 64 with a bias shared by the batch and key lengths: workgroups run
    # two batches each, paired by key-length rank (longest with shortest)
    g = torch.Generator().manual_seed(19)
    H, Nq, Nk, d = 2, 130, 300, 64
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    if lens is None:
        lens = torch.randint(0, Nk + 40, (B,), generator=g).tolist()  # some past Nk
    kv_len = torch.tensor(lens, dtype=torch.int32)
    bias = torch.randn(1, H, Nq, Nk, generator=g) * 0.5
    inp = {"q": q, "k": k, "v": v, "bias": bias, "kv_len": kv_len, "causal": False,
           "scale": 0.125}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"paired batches B={B}")


def test_no_keys_at_all():
    q = torch.randn(2, 2, 40, 64).to(torch.bfloat16)
    k = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16)
    o, lse = ea.attn_fwd(q.cuda(), k.cuda(), k.cuda())
    torch.cuda.synchronize()
    assert torch.all(o.cpu() == 0) and torch.all(torch.isneginf(lse.cpu()))


@pytest.mark.parametrize("hk", [1, 2])
def test_grouped_kv_heads(hk):
    # query head h reads key/value head h // (H / Hk)
    g = torch.Generator().manual_seed(12)
    B, H, N, d = 2, 4, 190, 128
    q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, hk, N, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, hk, N, d, generator=g).to(torch.bfloat16)
    o, lse = ea.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    rep = H // hk
    kx = k.repeat_interleave(rep, dim=1)
    vx = v.repeat_interleave(rep, dim=1)
    ro, rl = oracle.attention_forward(q.double().numpy(), kx.double().numpy(),
                                      vx.double().numpy(), scale=1 / math.sqrt(d),
                                      causal=True)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16",
            f"gqa Hk={hk}")


def test_strided_views():
    # [B, N, H, d] storage viewed as [B, H, N, d]; output written into a view
    g = torch.Generator().manual_seed(13)
    B, H, N, d = 2, 3, 211, 64
    base = torch.randn(3, B, N, H, d, generator=g).to(torch.bfloat16).cuda()
    q, k, v = (base[i].transpose(1, 2) for i in range(3))
    out_store = torch.empty(B, N, H, d, dtype=torch.bfloat16, device="cuda")
    out = out_store.transpose(1, 2)
    lse_store = torch.empty(B, H, N + 8, dtype=torch.float32, device="cuda")
    lse = lse_store[:, :, :N]
    ea.attn_fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward(q.double().cpu().numpy(), k.double().cpu().numpy(),
                                      v.double().cpu().numpy(), scale=1 / 8, causal=True)
    compare(out.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16", "strided")


def test_large_magnitude_scores():
    # scores near +-1e3 would overflow exp() without the running maximum
    g = torch.Generator().manual_seed(14)
    q = (torch.randn(1, 2, 130, 64, generator=g) * 30).to(torch.bfloat16)
    k = (torch.randn(1, 2, 130, 64, generator=g) * 30).to(torch.bfloat16)
    v = torch.randn(1, 2, 130, 64, generator=g).to(torch.bfloat16)
    inp = {"q": q, "k": k, "v": v, "bias": None, "kv_len": None, "causal": False,
           "scale": 0.125}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    assert np.abs(rl).max() > 500
    compare(o, lse, ro, rl, "bf16", "large scores")


@pytest.mark.parametrize("causal", [False, True])
def test_reference_jumps_between_tiles(causal):
    # Every key tile's scores lie about 40 base-2 units above the previous
    # tile's, so each tile overflows the kernel's probability-sum guard (2^32)
    # and takes the rare path that moves the reference; the result must not
    # change (any reference gives the same softmax).
    g = torch.Generator().manual_seed(16)
    nq, nk, d, scale = 70, 330, 64, 0.125
    q = torch.randn(1, 2, nq, d, generator=g) * 0.05
    q[..., 0] = 8.0
    k = torch.randn(1, 2, nk, d, generator=g) * 0.05
    step = 40.0 / (8.0 * scale * math.log2(math.e))  # raw k[...,0] per tile
    k[..., 0] = (torch.arange(nk) // 64).float() * step
    v = torch.randn(1, 2, nk, d, generator=g)
    inp = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16),
           "bias": None, "kv_len": None, "causal": causal, "scale": scale}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    compare(o, lse, ro, rl, "bf16", f"reference jumps causal={causal}")


def test_first_tile_masked_and_low_scores():
    # Rows 0..9 see nothing in the first key tile (-inf bias) and every other
    # key carries a bias of -300: a reference left at 0 would underflow all
    # their probabilities, so the kernel must set the reference from the first
    # tile that has a visible key.
    g = torch.Generator().manual_seed(17)
    nq, nk, d = 70, 200, 64
    q = torch.randn(1, 2, nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 2, nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 2, nk, d, generator=g).to(torch.bfloat16)
    bias = torch.full((1, 2, nq, nk), -300.0)
    bias[:, :, :10, :64] = -math.inf
    inp = {"q": q, "k": k, "v": v, "bias": bias, "kv_len": None, "causal": False,
           "scale": 0.125}
    o, lse = run_gpu(inp)
    ro, rl = run_oracle(inp)
    assert np.all(np.isfinite(rl)) and rl.max() < -200
    compare(o, lse, ro, rl, "bf16", "first tile masked, low scores")


def test_deterministic_bitwise():
    w = workloads.small("c3_bf16_d128_causal", B=1, H=4, Nq=777, Nk=777)
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    o1, l1 = ea.attn_fwd(q, k, v, causal=True)
    o2, l2 = ea.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_merge_of_two_key_halves_gpu():
    # FlashAttention: Mathematical Foundations..., section 7: two GPU calls on
    # disjoint key ranges, merged by their LSEs, reproduce the full call.
    g = torch.Generator().manual_seed(15)
    q = torch.randn(2, 2, 260, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, 2, 500, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, 2, 500, 128, generator=g).to(torch.bfloat16).cuda()
    o, lse = ea.attn_fwd(q, k, v)
    oa, la = ea.attn_fwd(q, k[:, :, :192], v[:, :, :192])
    ob, lb = ea.attn_fwd(q, k[:, :, 192:], v[:, :, 192:])
    torch.cuda.synchronize()
    f = lambda t: t.double().cpu().numpy()
    om, lm = oracle.merge_partials([(f(oa), f(la)), (f(ob), f(lb))])
    assert np.abs(om - f(o)).max() <= 2e-2
    assert np.abs(lm - f(lse)).max() <= 1e-3


def test_error_status_raises():
    q = torch.randn(1, 1, 16, 96, device="cuda").to(torch.bfloat16)
    with pytest.raises(ea.AttnError, match="UNSUPPORTED"):
        ea.attn_fwd(q, q, q)
    q = torch.randn(1, 1, 16, 64, device="cuda").to(torch.bfloat16)
    with pytest.raises(ea.AttnError, match="UNSUPPORTED"):
        ea.attn_fwd(q, q, q, scale=-1.0)
    with pytest.raises(ea.AttnError, match="INVALID"):
        ea.attn_fwd(q, q, q, scale=float("nan"))


# --------------------------------------------------------------- full-size workloads
#
# The full-size workloads run in the launch configuration the benchmark
# times. The outputs are pre-filled with NaN, so a row that no workgroup
# wrote cannot pass as a stale value of an earlier call; every row must come
# back finite. Then one row of every (batch, head, 128-row query tile) -- a
# different offset inside each tile, so the rows fall on every wavefront and
# lane position -- and every row of the first and the last head are compared
# with the oracle element by element. 128 rows is the smallest workgroup any
# launch uses, so every workgroup of every launch has at least one row
# checked. [flash-attention (stanleyjacob.dev), Part XII, testing against a
# slow reference.]

TILE_ROWS = 128


def nan_outputs(B, H, Nq, d, dtype):
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((B, H, Nq, d), float("nan"), dtype=st, device="cuda")
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


def tile_rows(B, H, Nq, seed, tile=TILE_ROWS):
    """One row per (b, h, query tile), at a seeded offset inside the tile."""
    r = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(H):
            for t0 in range(0, Nq, tile):
                rows.append((b, h, t0 + int(r.integers(min(tile, Nq - t0)))))
    return rows


def head_rows(b, h, Nq):
    return [(b, h, i) for i in range(Nq)]


def assert_all_written(o_c, lse_c, what):
    """Every row was written: no NaN left of the pre-fill anywhere."""
    assert not torch.isnan(o_c.float()).any(), f"{what}: O rows left unwritten (NaN)"
    assert not torch.isnan(lse_c).any(), f"{what}: LSE rows left unwritten (NaN)"


def compare_rows(o_c, lse_c, rows, oracle_rows, dtype, what, chunk=2048):
    """Compare the listed rows of a full-size output with the oracle, in
    chunks of rows so that one head of 16K keys stays within memory.
    oracle_rows(rows) returns (O [n, d], LSE [n]) in fp64."""
    for c0 in range(0, len(rows), chunk):
        part = rows[c0:c0 + chunk]
        ro, rl = oracle_rows(part)
        go = np.stack([o_c[b, h, i].double().numpy() for b, h, i in part])
        gl = np.array([float(lse_c[b, h, i]) for b, h, i in part])
        compare(go, gl, ro, rl, dtype, f"{what} rows {c0}..{c0 + len(part) - 1}")


def full_size_rows(w):
    """One row of every query tile, then all rows of the first and last head."""
    return (tile_rows(w.B, w.H, w.Nq, w.seed) + head_rows(0, 0, w.Nq)
            + head_rows(w.B - 1, w.H - 1, w.Nq))


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_full_size_every_tile(name):
    w = workloads.CONFIGS[name]
    _banner(f"full {name}")
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    bias = _to_gpu(inp["bias"])
    kv_len = _to_gpu(inp["kv_len"])
    o, lse = nan_outputs(w.B, w.H, w.Nq, w.d, w.dtype)
    ea.attn_fwd(q, k, v, bias=bias, kv_len=kv_len, causal=w.causal, scale=inp["scale"],
                out=o, lse=lse)
    torch.cuda.synchronize()
    o_c = o.cpu()
    lse_c = lse.cpu()
    assert_all_written(o_c, lse_c, name)
    # every configured row sees at least one key
    assert torch.isfinite(lse_c).all()
    # each O row inside the range of V (any size)
    vmin = inp["v"].float().amin(dim=2, keepdim=True)
    vmax = inp["v"].float().amax(dim=2, keepdim=True)
    slack = 1e-2 * (vmax - vmin) + 1e-6
    assert bool(((o_c.float() >= vmin - slack) & (o_c.float() <= vmax + slack)).all())
    f = lambda t: None if t is None else t.double().numpy()
    kv = None if inp["kv_len"] is None else inp["kv_len"].numpy()
    qd, kd, vd, bd = f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["bias"])

    def oracle_rows(part):
        return oracle.attention_rows(qd, kd, vd, part, scale=inp["scale"], bias=bd,
                                     kv_len=kv, causal=w.causal)

    compare_rows(o_c, lse_c, full_size_rows(w), oracle_rows, w.dtype, f"full {name}")


# Causal launches deal the flat heads in groups (longest query tiles of a
# whole group first). Shapes with several groups and a smaller last group,
# compared in full: d = 128 (256-row tiles, 4 per head, groups of 8 heads:
# 8 + 7) and d = 64 (128-row tiles, 8 per head, groups of 8: 8 + 8 + 5).
@pytest.mark.parametrize("d,B,H", [(128, 3, 5), (64, 3, 7)])
def test_causal_grouped_dispatch_ragged_last_group(d, B, H):
    w = workloads.Workload("grouped", B, H, 1000, 1000, d, causal=True, seed=31 + d)
    inp = workloads.make_inputs(w)
    o, lse = nan_outputs(B, H, 1000, d, "bf16")
    _banner(f"causal grouped dispatch d={d} B={B} H={H}")
    ea.attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), causal=True,
                scale=inp["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = run_oracle(inp)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16",
            f"causal grouped d={d} B={B} H={H}")


def _random_forward_cases(n, seed):
    """Seeded small problems through the per-tile kernels (too few query tiles
    for the persistent form): both dtypes and head dimensions, grouped K/V
    heads, causal or not, a bias broadcast over batches and/or heads, per-batch
    key lengths (zero and past Nk included), ragged counts."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        dtype = "f32" if r.random() < 0.25 else "bf16"
        d = int(r.choice([64, 128]))
        B = int(r.integers(1, 4))
        Hk = int(r.choice([1, 2]))
        H = Hk * int(r.choice([1, 2, 3]))
        Nq = int(r.integers(1, 700))
        Nk = int(r.integers(1, 700))
        causal = bool(r.integers(2))
        bias = None
        if r.random() < 0.5:
            bias = (int(r.choice([1, B])), int(r.choice([1, H])))
        kv = [int(x) for x in r.integers(0, Nk + 30, B)] if r.random() < 0.5 else None
        cases.append((dtype, d, B, H, Hk, Nq, Nk, causal, bias, kv))
    return cases


@pytest.mark.parametrize("dtype,d,B,H,Hk,Nq,Nk,causal,bias,kv", _random_forward_cases(12, 7373))
def test_random_small_problems(dtype, d, B, H, Hk, Nq, Nk, causal, bias, kv):
    # seeded problems, every row compared with the oracle [Understanding
    # FlashAttention Pt 1, sections 0.2, 2.4 and 3.5]
    _banner(f"random dtype={dtype} d={d} B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} causal={causal} "
            f"bias={bias} kv={kv}")
    g = torch.Generator().manual_seed(17 * Nq + Nk + d + B)
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(B, H, Nq, d, generator=g).to(st)
    k = torch.randn(B, Hk, Nk, d, generator=g).to(st)
    v = torch.randn(B, Hk, Nk, d, generator=g).to(st)
    bb = None if bias is None else 0.5 * torch.randn(bias[0], bias[1], Nq, Nk, generator=g)
    kl = None if kv is None else torch.tensor(kv, dtype=torch.int32)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    inp = {"q": q, "k": k, "v": v, "bias": bb, "kv_len": kl, "causal": causal, "scale": scale}
    o, lse = run_gpu(inp)
    rep = H // Hk
    ref = dict(inp)
    ref["k"] = k.repeat_interleave(rep, dim=1)
    ref["v"] = v.repeat_interleave(rep, dim=1)
    ro, rl = run_oracle(ref)
    compare(o, lse, ro, rl, dtype, f"random Nq={Nq} Nk={Nk}")
