"""Parity of the persistent ("stream") forward with the fp64 oracle.

Dense and causal bf16 problems (no bias, no key lengths, no window) whose
key count is a multiple of 128 and which have at least two 256-row query
tiles per compute unit run on one workgroup per compute unit that walks its
query tiles back to back: the next tile's Q rows are copied into LDS during the current tile,
the key/value stream runs across the boundary and the finished O leaves
through LDS during the next tile. The cases below all take that path (the
launcher picks it for these shapes) with several tiles per workgroup, an
uneven number of tiles per workgroup, ragged last query tiles, unequal query
and key counts, grouped key/value heads and strided views. Outputs start as
NaN; one row of every 128-row query tile and every row of the first and last
head are compared with the oracle at the parity bars. [Understanding
FlashAttention Pt 1, sections 2.4 and 3.1; FlashAttention: Mathematical
Foundations..., section 5.]
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_io_aware_06_amd as ea

from tests.test_gpu_parity import (_banner, assert_all_written, compare_rows, head_rows,
                                   nan_outputs, tile_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("these tests need a GPU")
    ea.load_library()
    yield


CASES = [
    # (B, H, Hk, Nq, Nk, d): tiles per head x heads >= 2 x 256
    (2, 96, 96, 1000, 1024, 128),    # 768 tiles: 3 per workgroup, ragged last tile
    (3, 68, 17, 700, 512, 64),       # grouped heads (4 per K/V head), 612 tiles
    (2, 101, 101, 1024, 896, 128),   # 808 tiles: 3 or 4 per workgroup, Nk = 14 tiles
    (1, 128, 128, 1300, 2048, 64),   # Nq > multiple of 256, long keys (128-key tiles)
]


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d", CASES)
def test_stream_matches_oracle(B, H, Hk, Nq, Nk, d):
    _banner(f"stream B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d}")
    w = workloads.Workload("stream", B, H, Nq, Nk, d, seed=B * H + Nq + Nk + d, Hk=Hk)
    inp = workloads.make_inputs(w)
    o, lse = nan_outputs(B, H, Nq, d, "bf16")
    ea.attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), scale=inp["scale"],
                out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream")
    rep = H // Hk
    f = lambda t: t.double().numpy()
    qd, kd, vd = f(inp["q"]), f(inp["k"]), f(inp["v"])

    def oracle_rows(part):
        out_o, out_l = [], []
        for b, h, i in part:
            oo, ll = oracle.attention_rows(qd[b:b + 1, h:h + 1], kd[b:b + 1, h // rep:h // rep + 1],
                                           vd[b:b + 1, h // rep:h // rep + 1], [(0, 0, i)],
                                           scale=inp["scale"])
            out_o.append(oo[0])
            out_l.append(ll[0])
        return np.stack(out_o), np.array(out_l)

    rows = tile_rows(B, H, Nq, w.seed) + head_rows(0, 0, Nq) + head_rows(B - 1, H - 1, Nq)
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", f"stream d={d} Nq={Nq} Nk={Nk}")


CAUSAL_CASES = [
    # (B, H, Hk, Nq, Nk, d): causal, Nk - Nq a multiple of 128, B*H a
    # multiple of 8, at least 512 query tiles
    (1, 64, 64, 1920, 2048, 128),   # diagonal offset 128, ragged last query tile
    (2, 32, 8, 2048, 2048, 64),     # grouped heads (4 per K/V head), offset 0
    (1, 64, 16, 2048, 2304, 64),    # offset 256, grouped heads
    # offset 0 at d = 128: a workgroup's last tile can have 4 key tiles,
    # fewer than the iterations that drain the previous tile's O
    (2, 32, 32, 2048, 2048, 128),
    # many heads per XCD: eight rounds, short tiles (4, 8, 12 key tiles)
    # back to back, each draining and copying at its start
    (8, 64, 64, 1024, 1024, 128),
    (4, 32, 8, 1024, 1152, 64),     # grouped heads, offset 128, short first tiles
]


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d", CAUSAL_CASES)
def test_stream_causal_matches_oracle(B, H, Hk, Nq, Nk, d):
    # Causal problems of these shapes take the persistent form with its
    # longest-first rounds; every row of three whole heads (every position
    # against the diagonal, in the first, a middle and the last head) and one
    # row of every 128-row tile are compared. [Understanding FlashAttention
    # Pt 1, section 3.5: causal tiles.]
    _banner(f"stream causal B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d}")
    w = workloads.Workload("stream_causal", B, H, Nq, Nk, d, causal=True,
                           seed=3 * B * H + Nq + Nk + d, Hk=Hk)
    inp = workloads.make_inputs(w)
    o, lse = nan_outputs(B, H, Nq, d, "bf16")
    ea.attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), scale=inp["scale"],
                causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream causal")
    rep = H // Hk
    f = lambda t: t.double().numpy()
    qd, kd, vd = f(inp["q"]), f(inp["k"]), f(inp["v"])

    def oracle_rows(part):
        out_o, out_l = [], []
        for b, h, i in part:
            oo, ll = oracle.attention_rows(qd[b:b + 1, h:h + 1], kd[b:b + 1, h // rep:h // rep + 1],
                                           vd[b:b + 1, h // rep:h // rep + 1], [(0, 0, i)],
                                           scale=inp["scale"], causal=True)
            out_o.append(oo[0])
            out_l.append(ll[0])
        return np.stack(out_o), np.array(out_l)

    rows = (tile_rows(B, H, Nq, w.seed) + head_rows(0, 0, Nq) + head_rows(B - 1, H // 2, Nq)
            + head_rows(B - 1, H - 1, Nq))
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", f"stream causal d={d} Nq={Nq} Nk={Nk}")


WINDOW_CASES = [
    # (B, H, Hk, Nq, Nk, d, causal, (left, right)): Nk >= Nq, at least 512
    # query tiles; bands of whole and partial tiles, made even
    (2, 64, 64, 1024, 1024, 128, True, (300, 0)),      # causal window, 6-7 key tiles
    (2, 64, 16, 1024, 1280, 64, False, (200, 100)),    # two-sided, offset 256, grouped heads
    (1, 128, 128, 1024, 1024, 128, False, (64, 37)),   # narrow band: short tiles copy at once
    (1, 64, 64, 2048, 2048, 128, True, (1100, 0)),     # 22-key-tile bands, spread copies
]


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal,window", WINDOW_CASES)
def test_stream_window_matches_oracle(B, H, Hk, Nq, Nk, d, causal, window):
    # Sliding windows on the persistent form with its rotated key order
    # (reading 18: key j kept iff i + Nk - Nq - left <= j <= i + Nk - Nq +
    # right); one row of every 128-row tile and three whole heads.
    # [flash-attention, Part III, window_size; FlashAttention, Explained,
    # section 14.]
    _banner(f"stream window B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d} causal={causal} {window}")
    w = workloads.Workload("stream_window", B, H, Nq, Nk, d, causal=causal, window=window,
                           seed=5 * B * H + Nq + Nk + d + window[0], Hk=Hk)
    inp = workloads.make_inputs(w)
    o, lse = nan_outputs(B, H, Nq, d, "bf16")
    ea.attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), scale=inp["scale"],
                causal=causal, window=window, out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream window")
    rep = H // Hk
    f = lambda t: t.double().numpy()
    qd, kd, vd = f(inp["q"]), f(inp["k"]), f(inp["v"])

    def oracle_rows(part):
        out_o, out_l = [], []
        for b, h, i in part:
            oo, ll = oracle.attention_rows(qd[b:b + 1, h:h + 1], kd[b:b + 1, h // rep:h // rep + 1],
                                           vd[b:b + 1, h // rep:h // rep + 1], [(0, 0, i)],
                                           scale=inp["scale"], causal=causal, window=window)
            out_o.append(oo[0])
            out_l.append(ll[0])
        return np.stack(out_o), np.array(out_l)

    rows = (tile_rows(B, H, Nq, w.seed) + head_rows(0, 0, Nq) + head_rows(B - 1, H // 2, Nq)
            + head_rows(B - 1, H - 1, Nq))
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", f"stream window {window}")


def test_stream_strided_views_and_determinism():
    # [B, N, H, d] storage seen as [B, H, N, d] for q, k, v and the output;
    # two calls are bitwise equal
    g = torch.Generator().manual_seed(71)
    B, H, N, d = 2, 128, 1024, 128
    base = torch.randn(3, B, N, H, d, generator=g).to(torch.bfloat16).cuda()
    q, k, v = (base[i].transpose(1, 2) for i in range(3))
    out_store = torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = out_store.transpose(1, 2)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    ea.attn_fwd(q, k, v, out=out, lse=lse)
    o2, l2 = ea.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    o_c, lse_c = out.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream strided")
    qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))

    def oracle_rows(part):
        return oracle.attention_rows(qd, kd, vd, part, scale=d ** -0.5)

    rows = tile_rows(B, H, N, 72) + head_rows(1, 77, N)
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", "stream strided")


def _random_stream_cases(n, seed):
    """Seeded shapes that meet the persistent form's conditions: at least
    two 256-row query tiles per compute unit (512 on MI355X's 256 CUs), key
    counts a multiple of 128; causal: Nk - Nq a multiple of 128 and B*H a
    multiple of 8; windows: Nk >= Nq. Tile counts per workgroup, ragged
    query tiles, diagonal offsets and band widths vary from case to case."""
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(r.choice([64, 128]))
        mode = ("dense", "causal", "window")[len(cases) % 3]
        rep = int(r.choice([1, 2, 4]))
        if mode == "causal":
            Nq = 128 * int(r.integers(4, 17))
            Nk = Nq + 128 * int(r.integers(0, 4))
        else:
            Nq = int(r.integers(200, 1700))
            Nk = 128 * int(r.integers(14 if d == 128 else 8, 21))
            if mode == "window":
                Nk = max(Nk, 128 * ((Nq + 127) // 128))
        tiles = (Nq + 255) // 256
        bh = int(r.integers(512, 1400)) // tiles + 1
        bh = max(8, ((bh + 8 * rep - 1) // (8 * rep)) * 8 * rep)   # B*H, a multiple of 8 * rep
        B = int(r.choice([b for b in (1, 2, 3, 4) if bh % (b * rep) == 0 and (bh // b) % 8 == 0] or [1]))
        H = bh // B
        if B * H * Nk * d > 80_000_000:
            continue
        causal, window = mode == "causal", None
        if mode == "window":
            causal = bool(r.integers(2))
            left = int(r.integers(1, 1500))
            right = 0 if causal else int(r.choice([-1, int(r.integers(0, 400))]))
            window = (left, right)
        cases.append((B, H, H // rep, Nq, Nk, d, causal, window))
    return cases


RANDOM_CASES = _random_stream_cases(12, 20260)


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,d,causal,window", RANDOM_CASES)
def test_stream_random_shapes(B, H, Hk, Nq, Nk, d, causal, window):
    # Seeded shapes across the persistent form's three deals (dense every
    # wpx-th tile, causal longest-first rounds, window rotated bands), with
    # grouped heads; one row of every 128-row tile and the first and last
    # heads in full. [Understanding FlashAttention Pt 1, sections 2.4, 3.1
    # and 3.5.]
    _banner(f"stream random B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} d={d} causal={causal} window={window}")
    w = workloads.Workload("stream_random", B, H, Nq, Nk, d, causal=causal, window=window,
                           seed=7 * B * H + 3 * Nq + Nk + d, Hk=Hk)
    inp = workloads.make_inputs(w)
    o, lse = nan_outputs(B, H, Nq, d, "bf16")
    ea.attn_fwd(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), scale=inp["scale"],
                causal=causal, window=window, out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream random")
    rep = H // Hk
    f = lambda t: t.double().numpy()
    qd, kd, vd = f(inp["q"]), f(inp["k"]), f(inp["v"])

    def oracle_rows(part):
        by_head = {}
        for n, (b, h, i) in enumerate(part):
            by_head.setdefault((b, h), []).append((n, i))
        out_o = np.zeros((len(part), d))
        out_l = np.zeros(len(part))
        for (b, h), items in by_head.items():
            oo, ll = oracle.attention_rows(qd[b:b + 1, h:h + 1], kd[b:b + 1, h // rep:h // rep + 1],
                                           vd[b:b + 1, h // rep:h // rep + 1],
                                           [(0, 0, i) for _, i in items], scale=inp["scale"],
                                           causal=causal, window=window)
            for r_, (n, _) in enumerate(items):
                out_o[n] = oo[r_]
                out_l[n] = ll[r_]
        return out_o, out_l

    rows = tile_rows(B, H, Nq, w.seed) + head_rows(0, 0, Nq) + head_rows(B - 1, H - 1, Nq)
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", f"stream random d={d} Nq={Nq} Nk={Nk}")


BIAS_CASES = [
    # (B, H, Hk, Nq, Nk, bias batches, bias heads, kv_len, -inf fraction):
    # d = 64, not causal, H a multiple of 8, at least 512 query tiles of 256
    # rows: padded batches with a bias on the persistent form
    (8, 16, 16, 1024, 1024, 1, 16, [614, 397, 242, 762, 429, 625, 464, 860], 0.0),
    (2, 64, 16, 1000, 700, 2, 64, [0, 700], 0.0),          # full bias, ragged rows, no keys
    (4, 32, 32, 1024, 516, 4, 1, None, 0.02),              # head-broadcast bias, -inf entries
    (2, 80, 20, 777, 1028, 1, 1, [1028, 3], 0.0),          # one bias for all; shifted last tile
    (4, 32, 8, 1024, 64, 1, 32, [1, 64, 63, 9999], 0.0),   # 64 keys (one tile), kv_len > Nk
    # 20 query rows: every wavefront's bias block re-reads the last row
    (8, 64, 64, 20, 300, 1, 64, [300, 1, 77, 0, 128, 129, 64, 299], 0.0),
]


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,bb,bh,kv,ninf", BIAS_CASES)
def test_stream_bias_matches_oracle(B, H, Hk, Nq, Nk, bb, bh, kv, ninf):
    # Additive fp32 bias (broadcast over batches and/or heads) and per-batch
    # key lengths on the persistent form (each wavefront's bias block copied
    # into LDS one key tile ahead): one row of every 128-row tile and the
    # first and last heads in full, NaN-filled outputs. [Understanding
    # FlashAttention Pt 1, section 0.2 (additive bias) and 3.5 (padding
    # masks); flash-attention, Part II (padded batches).]
    _banner(f"stream bias B={B} H={H} Hk={Hk} Nq={Nq} Nk={Nk} bias=[{bb},{bh}] kv={kv} ninf={ninf}")
    d = 64
    g = torch.Generator().manual_seed(B * H + Nq + Nk + bb + bh)
    q = torch.randn(B, H, Nq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hk, Nk, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hk, Nk, d, generator=g).to(torch.bfloat16)
    bias = 0.5 * torch.randn(bb, bh, Nq, Nk, generator=g)
    if ninf > 0:
        bias[torch.rand(bias.shape, generator=g) < ninf] = float("-inf")
        bias[0, 0, 5, :] = float("-inf")   # a row that sees no key at all
    kv_len = None if kv is None else torch.tensor(kv, dtype=torch.int32)
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    o, lse = nan_outputs(B, H, Nq, d, "bf16")
    ea.attn_fwd(q.cuda(), k.cuda(), v.cuda(), bias=bias.cuda(),
                kv_len=None if kv_len is None else kv_len.cuda(), scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream bias")
    rep = H // Hk
    f = lambda t: t.double().numpy()
    qd, kd, vd, bd = f(q), f(k), f(v), f(bias)
    kvn = None if kv_len is None else kv_len.numpy()

    def oracle_rows(part):
        by_head = {}
        for n, (b, h, i) in enumerate(part):
            by_head.setdefault((b, h), []).append((n, i))
        out_o = np.zeros((len(part), d))
        out_l = np.zeros(len(part))
        for (b, h), items in by_head.items():
            bsel = bd[(b if bb > 1 else 0):(b if bb > 1 else 0) + 1, (h if bh > 1 else 0):(h if bh > 1 else 0) + 1]
            oo, ll = oracle.attention_rows(qd[b:b + 1, h:h + 1], kd[b:b + 1, h // rep:h // rep + 1],
                                           vd[b:b + 1, h // rep:h // rep + 1],
                                           [(0, 0, i) for _, i in items], scale=scale, bias=bsel,
                                           kv_len=None if kvn is None else kvn[b:b + 1])
            for r_, (n, _) in enumerate(items):
                out_o[n] = oo[r_]
                out_l[n] = ll[r_]
        return out_o, out_l

    rows = tile_rows(B, H, Nq, B + H + Nq) + head_rows(0, 0, Nq) + head_rows(B - 1, H - 1, Nq)
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", f"stream bias Nq={Nq} Nk={Nk}")


def test_stream_bias_strided_views_and_determinism():
    # [B, N, H, d] storage seen as [B, H, N, d] for q, k, v and the output, a
    # bias whose rows are padded to a larger stride, key lengths; the biased
    # persistent form (d = 64) against the oracle, and two calls bitwise equal
    g = torch.Generator().manual_seed(97)
    B, H, N, Nk, d = 4, 32, 1024, 640, 64
    qs = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).cuda()
    ks = torch.randn(B, Nk, H, d, generator=g).to(torch.bfloat16).cuda()
    vs = torch.randn(B, Nk, H, d, generator=g).to(torch.bfloat16).cuda()
    q, k, v = qs.transpose(1, 2), ks.transpose(1, 2), vs.transpose(1, 2)
    bias_store = 0.5 * torch.randn(1, H, N, Nk + 12, generator=g)
    bias = bias_store[..., :Nk].cuda()          # row stride Nk + 12 floats (16-byte multiple)
    kv_len = torch.tensor([640, 100, 513, 0], dtype=torch.int32)
    out_store = torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = out_store.transpose(1, 2)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    ea.attn_fwd(q, k, v, bias=bias, kv_len=kv_len.cuda(), out=out, lse=lse)
    o2, l2 = ea.attn_fwd(q, k, v, bias=bias, kv_len=kv_len.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    o_c, lse_c = out.cpu(), lse.cpu()
    assert_all_written(o_c, lse_c, "stream bias strided")
    qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))
    bd = bias.double().cpu().numpy()

    def oracle_rows(part):
        return oracle.attention_rows(qd, kd, vd, part, scale=d ** -0.5, bias=bd, kv_len=kv_len.numpy())

    rows = tile_rows(B, H, N, 98) + head_rows(1, 17, N) + head_rows(3, 0, N)
    compare_rows(o_c, lse_c, rows, oracle_rows, "bf16", "stream bias strided")


def _random_bias_cases(n, seed):
    """Seeded padded batches with a bias that take the biased persistent
    form: d = 64, H a multiple of 8, at most 64 batches, Nk a multiple of 4
    and at least 64, at least 512 query tiles of 256 rows; bias broadcast
    over batches and/or heads or not, key lengths drawn per batch (some
    zero, some beyond Nk) or absent."""
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        Nq = int(r.integers(100, 1300))
        Nk = 4 * int(r.integers(16, 400))
        tiles = (Nq + 255) // 256
        B = int(r.integers(1, 9))
        H = 8 * max(1, -(-512 // (8 * B * tiles)) + int(r.integers(0, 3)))
        if B * H * Nk * 64 > 60_000_000 or B * H * Nq * Nk > 4_000_000_000:
            continue
        Hk = H // int(r.choice([h for h in (1, 2, 4, 8) if H % h == 0]))
        bb = B if r.random() < 0.5 else 1
        bh = H if r.random() < 0.7 else 1
        kv = None
        if r.random() < 0.8:
            kv = [int(x) for x in r.integers(0, Nk + 100, B)]
        cases.append((B, H, Hk, Nq, Nk, bb, bh, kv, 0.0))
    return cases


@pytest.mark.parametrize("B,H,Hk,Nq,Nk,bb,bh,kv,ninf", _random_bias_cases(6, 4242))
def test_stream_bias_random_shapes(B, H, Hk, Nq, Nk, bb, bh, kv, ninf):
    # seeded shapes through the same checks as the fixed biased cases
    test_stream_bias_matches_oracle(B, H, Hk, Nq, Nk, bb, bh, kv, ninf)
