"""Parity of the packed variable-length forward with the oracle.

attn_fwd_varlen on token-major packed tensors against the oracle's
``attention_varlen`` (plain attention per sequence) on the same seeded
bytes, at the bars of the other parity tests. Cases: empty sequences, one-
row sequences, lengths that span several tiles with ragged tails, causal
and not, both head dimensions and dtypes, grouped K/V heads, different query
and key offsets per sequence (bottom-right causal alignment per sequence),
a window, rows past the last sequence left untouched, a generous
max_seqlen_q, offsets outside the tensors (clamped: no access leaves them),
and the packed workload at full size (one row of every query tile and
whole sequences, into NaN-filled outputs). [flash-attention
(stanleyjacob.dev), Part II "Variable-length batches: stop padding", Lab 5.]
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


def _packed(lens_q, lens_k, H, Hk, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    cu_q = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    q = torch.randn(int(cu_q[-1]), H, d, generator=g).to(st)
    k = torch.randn(int(cu_k[-1]), Hk, d, generator=g).to(st)
    v = torch.randn(int(cu_k[-1]), Hk, d, generator=g).to(st)
    return q, k, v, cu_q, cu_k


def _run(q, k, v, cu_q, cu_k, max_q, causal, window=None, scale=None, out=None, lse=None):
    o, l = ea.attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), max_q,
                              causal=causal, window=window, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


CASES = [
    # (lens_q, lens_k, H, Hk, d, dtype, causal)
    ([300, 1, 0, 513, 64, 1000], None, 2, 2, 128, "bf16", True),
    ([300, 1, 0, 513, 64, 1000], None, 2, 2, 64, "bf16", False),
    ([257, 700, 5], None, 4, 1, 128, "bf16", True),          # grouped K/V heads
    ([17, 200], [90, 650], 2, 2, 64, "bf16", True),          # fewer queries than keys
    ([40, 3], [10, 0], 2, 2, 128, "bf16", False),            # a sequence without keys
    ([129, 31, 260], None, 2, 2, 64, "f32", True),
    ([70, 200], [100, 150], 2, 1, 128, "f32", False),
]


@pytest.mark.parametrize("lens_q,lens_k,H,Hk,d,dtype,causal", CASES)
def test_varlen_matches_oracle(lens_q, lens_k, H, Hk, d, dtype, causal):
    lens_k = lens_q if lens_k is None else lens_k
    _banner(f"varlen q={lens_q} k={lens_k} H={H} Hk={Hk} d={d} {dtype} causal={causal}")
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hk, d, dtype, seed=sum(lens_q) + d)
    o, lse = _run(q, k, v, cu_q, cu_k, max(lens_q), causal)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=d ** -0.5, causal=causal)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy().T, ro, rl.T, dtype,
            f"varlen {lens_q}")


# Packed sequences with H a multiple of 8, at most 64 sequences and at least
# 64 keys in all take the persistent kernel (one workgroup per compute unit
# walking a longest-first list of (sequence, head, query tile) built on the
# device, 64-key tiles read shifted at a sequence's end and masked to the
# sequence's own keys). Cases: empty, one-row and sub-64-key sequences, a
# sequence without keys, more queries than keys (rows that see no key),
# grouped K/V heads, many short sequences, long ones of several query tiles.
PERSISTENT_CASES = [
    # (lens_q, lens_k, H, Hk, d, causal)
    ([300, 1, 0, 513, 64, 1000], None, 8, 8, 128, True),
    ([300, 1, 0, 513, 64, 1000], None, 8, 8, 64, False),
    ([257, 700, 5], None, 16, 2, 128, True),
    ([17, 200], [90, 650], 8, 8, 64, True),
    ([40, 3, 100], [10, 0, 80], 8, 8, 128, False),
    ([40, 3, 100], [10, 0, 80], 8, 4, 64, True),
    ([300, 200, 129], [100, 250, 129], 8, 8, 128, True),
    ([2100, 1300, 64, 65, 777], None, 8, 2, 128, True),
    ([2100, 1300, 64, 65, 777], None, 8, 8, 64, False),
    ([5, 61, 130, 255, 256, 257, 1, 90, 300, 12, 44, 199, 63, 64, 65, 511, 512, 513, 7, 100,
      20, 380, 3, 33, 250], None, 8, 8, 64, True),
    ([5, 61, 130, 255, 256, 257, 1, 90, 300, 12, 44, 199, 63, 64, 65, 511, 512, 513, 7, 100,
      20, 380, 3, 33, 250], [64, 10, 130, 700, 0, 257, 1, 90, 300, 500, 44, 199, 63, 64, 65,
                             511, 100, 513, 7, 100, 20, 380, 3, 33, 250], 8, 8, 128, False),
    ([700, 33, 1200], [900, 33, 1000], 8, 1, 128, True),    # one K/V head for all
    ([700, 33, 1200], None, 16, 1, 64, False),
]


@pytest.mark.parametrize("lens_q,lens_k,H,Hk,d,causal", PERSISTENT_CASES)
def test_varlen_persistent_matches_oracle(lens_q, lens_k, H, Hk, d, causal):
    lens_k = lens_q if lens_k is None else lens_k
    _banner(f"varlen persistent q={lens_q} k={lens_k} H={H} Hk={Hk} d={d} causal={causal}")
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hk, d, "bf16", seed=3 * sum(lens_q) + d)
    T = q.shape[0]
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = _run(q, k, v, cu_q, cu_k, max(lens_q), causal, out=out, lse=lse)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=d ** -0.5, causal=causal)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy().T, ro, rl.T, "bf16",
            f"varlen persistent {lens_q}")


@pytest.mark.parametrize("case", ["max_seqs", "alternating_deal", "table_limit", "per_tile_65"])
def test_varlen_persistent_limits(case):
    # the persistent form's limits: 64 sequences (the most it takes), more
    # than 16 items per workgroup (the alternating deal instead of the
    # greedy one: 64 sequences x 5 query tiles x 2 heads per XCD), the
    # largest tile list (64 sequences x ceil(8192 / 256) = 2048 entries), and
    # 65 sequences (the per-tile launch); compared in full
    r = np.random.default_rng({"max_seqs": 1, "alternating_deal": 2, "table_limit": 3,
                               "per_tile_65": 4}[case])
    if case == "max_seqs":
        lens, H, Hk, d, causal, max_q = list(r.integers(1, 400, 64)), 8, 8, 64, True, None
    elif case == "alternating_deal":
        lens, H, Hk, d, causal, max_q = list(r.integers(1030, 1100, 64)), 16, 8, 64, True, None
    elif case == "table_limit":
        lens, H, Hk, d, causal, max_q = list(r.integers(1, 90, 64)), 8, 2, 128, False, 8192
        lens[17] = 1500
    else:
        lens, H, Hk, d, causal, max_q = list(r.integers(1, 300, 65)), 8, 8, 128, True, None
    lens = [int(x) for x in lens]
    _banner(f"varlen persistent limits {case}: {len(lens)} sequences, {sum(lens)} rows, H={H}")
    q, k, v, cu_q, cu_k = _packed(lens, lens, H, Hk, d, "bf16", seed=sum(lens))
    T = q.shape[0]
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = _run(q, k, v, cu_q, cu_k, max_q or max(lens), causal, out=out, lse=lse)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=d ** -0.5, causal=causal)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy().T, ro, rl.T, "bf16",
            f"varlen persistent limits {case}")


def test_varlen_persistent_offsets_outside_tensors_are_clamped():
    # the clamped-offsets case of the per-tile kernel, with 8 heads (the
    # persistent kernel): [0, 120), an empty sequence and [80, 200)
    q, k, v, _, _ = _packed([200], [200], 8, 8, 128, "bf16", seed=64)
    cu = torch.tensor([-7, 120, 80, 1 << 30], dtype=torch.int32)
    o, l = _run(q, k, v, cu, cu, 256, True)
    oc, lc = o.cpu().double().numpy(), l.cpu().double().numpy().T
    assert not np.isnan(oc).any()
    f = lambda t: t.double().numpy()
    for lo, hi, keep in ((0, 120, np.r_[0:80]), (80, 200, np.r_[120:200])):
        ro, rl = oracle.attention_varlen(f(q), f(k), f(v), np.array([lo, hi]), np.array([lo, hi]),
                                         scale=128 ** -0.5, causal=True)
        compare(oc[keep], lc[keep], ro[keep], rl.T[keep], "bf16",
                f"varlen persistent clamped offsets [{lo}, {hi})")


def test_varlen_window():
    lens = [900, 77, 600]
    q, k, v, cu_q, cu_k = _packed(lens, lens, 2, 2, 128, "bf16", seed=61)
    for causal, window in ((True, (150, 0)), (False, (64, 100))):
        _banner(f"varlen window causal={causal} window={window}")
        o, lse = _run(q, k, v, cu_q, cu_k, max(lens), causal, window=window)
        ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(),
                                         v.double().numpy(), cu_q.numpy(), cu_k.numpy(),
                                         scale=128 ** -0.5, causal=causal, window=window)
        compare(o.double().cpu().numpy(), lse.double().cpu().numpy().T, ro, rl.T, "bf16",
                f"varlen window {window}")


def test_varlen_rows_outside_sequences_untouched_and_generous_max():
    # the sequences cover rows [0, 400) of 420 packed rows (offsets are
    # contiguous, so rows past the last offset are the only uncovered ones);
    # those rows of o and lse keep their contents. The second sequence has
    # 50 rows and no keys (zero rows, -inf LSE).
    q, k, v, _, _ = _packed([420], [420], 2, 2, 64, "bf16", seed=62)
    cu_q = torch.tensor([0, 250, 300, 400], dtype=torch.int32)
    cu_k = torch.tensor([0, 250, 250, 400], dtype=torch.int32)
    out = torch.full((420, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((2, 420), 7.0, dtype=torch.float32, device="cuda")
    o, l = _run(q, k, v, cu_q, cu_k, 4096, True, out=out, lse=lse)
    oc, lc = o.cpu(), l.cpu()
    assert torch.all(oc[400:] == 7.0) and torch.all(lc[:, 400:] == 7.0)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=0.125, causal=True)
    compare(oc.double().numpy()[:400], lc.double().numpy().T[:400], ro[:400], rl.T[:400],
            "bf16", "varlen partial cover")


def test_varlen_offsets_outside_tensors_are_clamped():
    # Offsets outside the packed tensors and a decreasing pair: the kernels
    # clamp each sequence to start = clamp(cu[s], 0, total), end =
    # clamp(cu[s+1], start, total), so every access stays inside the tensors.
    # Here that gives [0, 120), an empty sequence, and [80, 200); rows both
    # cover are unspecified, the rest follow the clamped sequences.
    q, k, v, _, _ = _packed([200], [200], 2, 2, 128, "bf16", seed=63)
    cu = torch.tensor([-7, 120, 80, 1 << 30], dtype=torch.int32)
    o, l = _run(q, k, v, cu, cu, 256, False)
    oc, lc = o.cpu().double().numpy(), l.cpu().double().numpy().T
    assert not np.isnan(oc).any()
    f = lambda t: t.double().numpy()
    for lo, hi, keep in ((0, 120, np.r_[0:80]), (80, 200, np.r_[120:200])):
        ro, rl = oracle.attention_varlen(f(q), f(k), f(v), np.array([lo, hi]), np.array([lo, hi]),
                                         scale=128 ** -0.5)
        compare(oc[keep], lc[keep], ro[keep], rl.T[keep], "bf16",
                f"varlen clamped offsets [{lo}, {hi})")


@pytest.mark.parametrize("name", sorted(workloads.VARLEN))
def test_varlen_full_size_every_tile(name):
    # NaN-filled outputs (the sequences cover every packed row, so every row
    # must come back written); one row of every (sequence, head, 128-row
    # query tile) and every row of the first and last sequence at the first
    # and last head against the oracle
    w = workloads.VARLEN[name]
    _banner(f"varlen full {name}")
    inp = workloads.make_varlen_inputs(w)
    cu = inp["cu"]
    T = inp["q"].shape[0]
    st = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.full((T, w.H, w.d), float("nan"), dtype=st, device="cuda")
    lse = torch.full((w.H, T), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = _run(inp["q"], inp["k"], inp["v"], cu, cu, inp["max_len"], w.causal,
                  scale=inp["scale"], out=out, lse=lse)
    oc, lc = o.cpu(), lse.cpu()
    assert not torch.isnan(oc.float()).any() and not torch.isnan(lc).any()
    assert torch.isfinite(lc).all()
    r = np.random.default_rng(w.seed)
    c = cu.tolist()
    rep = w.H // w.kv_heads
    picks = []   # (sequence, head, rows inside the sequence)
    for s in range(w.B):
        n = c[s + 1] - c[s]
        for h in range(w.H):
            picks.append((s, h, [t0 + int(r.integers(min(128, n - t0))) for t0 in range(0, n, 128)]))
    for s in (0, w.B - 1):
        n = c[s + 1] - c[s]
        for h in (0, w.H - 1):
            picks.append((s, h, list(range(n))))
    go, gl, ro, rl = [], [], [], []
    for s, h, idx in picks:
        f = lambda t, hh: t[c[s]:c[s + 1], hh].double().numpy()[None, None]
        oo, ll = oracle.attention_rows(f(inp["q"], h), f(inp["k"], h // rep), f(inp["v"], h // rep),
                                       [(0, 0, i) for i in idx], scale=inp["scale"],
                                       causal=w.causal)
        go.append(oc[[c[s] + i for i in idx], h].double().numpy())
        gl.append(lc[h, [c[s] + i for i in idx]].double().numpy())
        ro.append(oo)
        rl.append(ll)
    compare(np.concatenate(go), np.concatenate(gl), np.concatenate(ro), np.concatenate(rl),
            w.dtype, f"varlen full {name} every tile")


def _random_varlen_cases(n, seed):
    """Seeded packed batches: 1-64 sequences whose lengths mix lognormal
    draws with empty, single-row and tile-edge lengths, key lengths equal to
    the query lengths or drawn separately, H a multiple of 8 (the persistent
    form) with one to all query heads per K/V head."""
    r = np.random.default_rng(seed)
    edge = [0, 1, 63, 64, 65, 255, 256, 257]
    cases = []
    for c in range(n):
        ns = int(r.integers(1, 65))
        lq = [int(min(3000, round(float(np.exp(np.log(300) + 1.0 * r.normal())))))
              if r.random() < 0.8 else int(r.choice(edge)) for _ in range(ns)]
        lk = None
        if c % 3 == 2:
            lk = [int(min(3000, max(0, x + int(r.integers(-100, 300))))) for x in lq]
        H = int(r.choice([8, 16, 24]))
        Hk = int(r.choice([h for h in (1, 2, 4, 8, H) if H % h == 0]))
        d = int(r.choice([64, 128]))
        cases.append((lq, lk, H, Hk, d, bool(c % 2)))
    return cases


@pytest.mark.parametrize("lens_q,lens_k,H,Hk,d,causal", _random_varlen_cases(10, 9090))
def test_varlen_random_batches(lens_q, lens_k, H, Hk, d, causal):
    # seeded packed batches against the oracle, compared in full into
    # NaN-filled outputs [flash-attention, Part II, variable-length batches]
    lens_k = lens_q if lens_k is None else lens_k
    _banner(f"varlen random {len(lens_q)} sequences rows={sum(lens_q)} keys={sum(lens_k)} "
            f"H={H} Hk={Hk} d={d} causal={causal}")
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hk, d, "bf16", seed=5 * sum(lens_q) + d + H)
    T = q.shape[0]
    out = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = _run(q, k, v, cu_q, cu_k, max(max(lens_q), 1), causal, out=out, lse=lse)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=d ** -0.5, causal=causal)
    compare(o.double().cpu().numpy(), lse.double().cpu().numpy().T, ro, rl.T, "bf16",
            f"varlen random {len(lens_q)} sequences")


def _random_varlen_tile_cases(n, seed):
    """Seeded packed batches for the per-tile launch (H not a multiple of 8,
    or fp32): both dtypes and head dimensions, a window on some."""
    r = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        ns = int(r.integers(1, 20))
        lq = [int(min(1500, round(float(np.exp(np.log(200) + 1.0 * r.normal())))))
              if r.random() < 0.8 else int(r.choice([0, 1, 63, 64, 65, 256, 257])) for _ in range(ns)]
        lk = None
        if c % 3 == 1:
            lk = [int(min(1500, max(0, x + int(r.integers(-60, 200))))) for x in lq]
        Hk = int(r.choice([1, 2, 3]))
        H = Hk * int(r.choice([1, 2]))
        d = int(r.choice([64, 128]))
        dtype = "f32" if r.random() < 0.3 else "bf16"
        window = (int(r.integers(0, 300)), int(r.integers(-1, 100))) if r.random() < 0.3 else None
        cases.append((lq, lk, H, Hk, d, dtype, bool(c % 2), window))
    return cases


@pytest.mark.parametrize("lens_q,lens_k,H,Hk,d,dtype,causal,window", _random_varlen_tile_cases(8, 7171))
def test_varlen_random_tile_batches(lens_q, lens_k, H, Hk, d, dtype, causal, window):
    # seeded packed batches through the per-tile launch, compared in full
    # [flash-attention, Part II, variable-length batches]
    lens_k = lens_q if lens_k is None else lens_k
    _banner(f"varlen random tile {len(lens_q)} sequences rows={sum(lens_q)} keys={sum(lens_k)} "
            f"H={H} Hk={Hk} d={d} {dtype} causal={causal} window={window}")
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, H, Hk, d, dtype, seed=9 * sum(lens_q) + d + H)
    o, lse = _run(q, k, v, cu_q, cu_k, max(max(lens_q), 1), causal, window=window)
    ro, rl = oracle.attention_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     cu_q.numpy(), cu_k.numpy(), scale=d ** -0.5, causal=causal,
                                     window=window)
    T = q.shape[0]
    compare(o.double().cpu().numpy()[:T], lse.double().cpu().numpy().T[:T], ro, rl.T, dtype,
            f"varlen random tile {len(lens_q)} sequences")
