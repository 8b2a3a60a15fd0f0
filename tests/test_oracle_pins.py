"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties the oracle to one of: numbers printed on the pages (fixtures in
tests/golden), closed forms, invariants the mathematics fixes, an evaluation
in 50-digit decimal arithmetic, or a brute-force loop on tiny inputs that
takes a different route (no max subtraction). The mutation tests re-run these
functions against oracles with planted mistakes, so every test here must be
self-contained (no fixtures).
"""

import math
from decimal import Decimal, getcontext

import numpy as np

import oracle
from tests._golden import load


def _rng(seed):
    return np.random.default_rng(seed)


def _row_attention(scores, values):
    """Route a given score row through the full [B,H,N,d] oracle: one query
    (q = [1]), keys k_j = s_j, scale 1, so S = scores exactly."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    q = np.ones((1, 1, 1, 1))
    k = scores.reshape(1, 1, -1, 1)
    v = values.reshape(1, 1, len(scores), -1)
    o, lse = oracle.attention_forward(q, k, v, scale=1.0)
    return o[0, 0, 0], lse[0, 0, 0]


# ---------------------------------------------------------------- pages' numbers

def test_worked_row_two_blocks():
    g = load("worked_row_two_blocks.txt")
    tol = g["tol"]
    s, v = g["scores"], g["values"]
    o, lse = _row_attention(s, v)
    assert np.allclose(o, g["o"], atol=tol, rtol=0)
    # the denominator: LSE = max + ln(l)
    assert abs(math.exp(lse - s.max()) - g["l"]) < tol
    # block 1 alone gives m1, l1 and its accumulator a1 = [1, e^-1]
    o1, _, m1, l1 = oracle.online_softmax_blocked(s[:2], v[:2], int(g["block"]))
    assert m1 == g["m1"] and abs(l1 - g["l1"]) < tol
    assert np.allclose(o1 * l1, [1.0, math.exp(-1.0)], atol=1e-15)
    # both blocks: the accumulator before the final division, and the result
    ob, lseb, mb, lb = oracle.online_softmax_blocked(s, v, int(g["block"]))
    assert np.allclose(ob * lb, g["a2"], atol=tol, rtol=0)
    assert abs(lb - g["l"]) < tol and np.allclose(ob, g["o"], atol=tol, rtol=0)
    assert abs(lseb - lse) < 1e-14


def test_eight_scores_example():
    g = load("eight_scores.txt")
    tol = g["tol"]
    s, v = g["scores"], g["values"]
    o, lse = _row_attention(s, v)
    assert abs(o[0] - g["o"]) < tol
    p, m, l = oracle.masked_softmax(oracle.score_matrix(
        np.ones((1, 1)), s.reshape(-1, 1), 1.0))
    assert np.allclose(p[0], g["weights"], atol=g["weights_tol"], rtol=0)
    blk = int(g["block"])
    o1, _, m1, l1 = oracle.online_softmax_blocked(s[:blk], v[:blk], blk)
    assert m1 == g["m1"] and abs(l1 - g["l1"]) < tol
    assert abs(o1[0] * l1 - g["o_tilde1"]) < tol
    # the second block on its own, relative to the new maximum 7
    o2, _, m2, l2 = oracle.online_softmax_blocked(s[blk:], v[blk:], blk)
    assert m2 == 7 and abs(l2 - g["block2_sum"]) < tol
    assert abs(o2[0] * l2 - g["block2_times_v"]) < tol
    assert abs(math.exp(m1 - m2) - g["alpha"]) < tol
    ob, _, mb, lb = oracle.online_softmax_blocked(s, v, blk)
    assert abs(lb - g["l"]) < tol
    assert abs(ob[0] * lb - g["o_tilde"]) < g["o_tilde_tol"]
    assert abs(ob[0] - o[0]) < 1e-12


def test_lse_two_tiles():
    g = load("lse_two_tiles.txt")
    tol = g["tol"]
    s = g["scores"]
    v = np.eye(len(s))
    _, lse = _row_attention(s, v)
    assert abs(lse - g["lse"]) < g["lse_tol"]
    o1, _, m1, l1 = oracle.online_softmax_blocked(s[:2], v[:2], 2)
    assert m1 == g["m1"] and abs(l1 - g["l1"]) < tol
    _, lseb, mb, lb = oracle.online_softmax_blocked(s, v, int(g["block"]))
    assert abs(math.exp(m1 - mb) - g["correction"]) < tol
    assert abs(lb - g["l"]) < tol
    assert abs(mb + math.log(lb) - lse) < 1e-14


def test_causal_pattern_3x3():
    g = load("causal_3x3.txt")
    allowed = g["allowed"].astype(bool)
    r = _rng(1)
    q = r.normal(size=(1, 1, 3, 4))
    k = r.normal(size=(1, 1, 3, 4))
    s = oracle.score_matrix(q[0, 0], k[0, 0], 0.5, causal=True)
    assert np.array_equal(np.isfinite(s), allowed)
    p, _, _ = oracle.masked_softmax(s)
    assert np.all(p[~allowed] == 0.0)
    assert np.all(p[allowed] > 0.0)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-15)


def test_overflow_row():
    # Understanding FlashAttention Pt 1, §2.2: x = [1000, 999] must not
    # overflow; subtracting the maximum leaves [0, -1].
    o, lse = _row_attention([1000.0, 999.0], np.eye(2))
    e = math.exp(-1.0)
    assert np.allclose(o, [1 / (1 + e), e / (1 + e)], atol=1e-15, rtol=0)
    assert abs(lse - (1000.0 + math.log1p(e))) < 1e-12


# ---------------------------------------------------------------- invariants

def test_rows_sum_to_one_from_lse():
    # flash-attention, Lab 3: exp(s - LSE) over a row sums to 1.
    r = _rng(2)
    q = r.normal(size=(2, 3, 40, 16))
    k = r.normal(size=(2, 3, 56, 16))
    v = r.normal(size=(2, 3, 56, 8))
    bias = r.normal(size=(1, 3, 40, 56))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, scale=0.25, bias=bias,
                                          causal=causal)
        for b in range(2):
            for h in range(3):
                s = oracle.score_matrix(q[b, h], k[b, h], 0.25, bias[0, h],
                                        causal=causal)
                tot = np.exp(s - lse[b, h][:, None]).sum(axis=1)
                assert np.all(np.abs(tot - 1.0) <= 1e-12)


def test_row_shift_invariance():
    # Adding a constant c_i to every score of row i leaves O unchanged and
    # moves LSE_i by c_i (FlashAttention, Explained, §9).
    r = _rng(3)
    q = r.normal(size=(1, 2, 24, 8))
    k = r.normal(size=(1, 2, 31, 8))
    v = r.normal(size=(1, 2, 31, 5))
    c = r.normal(size=(1, 2, 24, 1)) * 30.0
    o0, l0 = oracle.attention_forward(q, k, v, scale=0.7)
    o1, l1 = oracle.attention_forward(q, k, v, scale=0.7,
                                      bias=np.broadcast_to(c, (1, 2, 24, 31)))
    assert np.allclose(o1, o0, atol=1e-12, rtol=0)
    assert np.allclose(l1, l0 + c[..., 0], atol=1e-11, rtol=0)


def test_scalar_recurrence_matches_definition():
    # Understanding FlashAttention Pt 1, §2.3: one key at a time.
    r = _rng(4)
    for n in (1, 2, 7, 100):
        s = r.normal(size=n) * 3
        v = r.normal(size=(n, 6))
        o, lse = _row_attention(s, v)
        o2, lse2, m2, l2 = oracle.online_softmax_scalar(s, v)
        assert np.allclose(o2, o, atol=1e-12, rtol=0)
        assert abs(lse2 - lse) <= 1e-12
        assert m2 == s.max()


def test_block_size_invariance():
    # "Understanding FlashAttention Pt 1", §2.4: the recurrence does not
    # depend on where the tile boundaries fall, and for a block of query rows
    # with masked (-inf) positions it is the direct masked softmax. Checked
    # against scipy's softmax / logsumexp on a 6-row block of 37 keys with
    # masked positions, one row with a single visible key and one row with
    # none, for block widths that split it evenly, raggedly, or not at all.
    from scipy.special import logsumexp, softmax
    r = _rng(11)
    s = 3.0 * r.normal(size=(6, 37))
    v = r.normal(size=(37, 3))
    s[1, ::3] = -np.inf           # every third key hidden
    s[2, :] = -np.inf
    s[2, 20] = 0.5                # a single visible key, in a middle block
    s[3, :] = -np.inf             # no visible key at all
    s[4, :30] = -np.inf           # only the last (ragged) block visible
    live = np.isfinite(s).any(axis=1)
    ref_o = np.zeros((6, 3))
    ref_lse = np.full(6, -np.inf)
    ref_o[live] = softmax(s[live], axis=1) @ v
    ref_lse[live] = logsumexp(s[live], axis=1)
    outs = []
    for blk in (1, 2, 5, 8, 36, 37, 100):
        o, lse, m, ell = oracle.online_softmax_blocked(s, v, blk)
        assert np.abs(o - ref_o).max() < 1e-13
        assert np.array_equal(np.isneginf(lse), ~live)
        assert np.abs(lse[live] - ref_lse[live]).max() < 1e-13
        assert np.array_equal(o[~live], np.zeros((int((~live).sum()), 3)))
        # the state's maximum is the row maximum; its sum is l = exp(lse - m)
        assert np.array_equal(m[live], s[live].max(axis=1))
        assert np.abs(ell[live] - np.exp(ref_lse[live] - m[live])).max() < 1e-12
        outs.append(o)
    # one row at a time gives the same rows
    for i in range(6):
        oi, lsei, _, _ = oracle.online_softmax_blocked(s[i], v, 4)
        assert np.abs(oi - ref_o[i]).max() < 1e-13
        assert (lsei == -np.inf) if not live[i] else abs(lsei - ref_lse[i]) < 1e-13


def test_merge_identity():
    # FlashAttention: Mathematical Foundations..., §7: partial (O, LSE) over
    # disjoint key ranges merge into the full result.
    r = _rng(5)
    q = r.normal(size=(2, 2, 9, 8))
    k = r.normal(size=(2, 2, 40, 8))
    v = r.normal(size=(2, 2, 40, 3))
    o, lse = oracle.attention_forward(q, k, v, scale=0.4)
    for cut in (1, 17, 39):
        pa = oracle.attention_forward(q, k[:, :, :cut], v[:, :, :cut], scale=0.4)
        pb = oracle.attention_forward(q, k[:, :, cut:], v[:, :, cut:], scale=0.4)
        om, lm = oracle.merge_partials([pa, pb])
        assert np.allclose(om, o, atol=1e-13, rtol=0)
        assert np.allclose(lm, lse, atol=1e-13, rtol=0)
    # three parts, and a part that is empty (all keys masked)
    parts = [oracle.attention_forward(q, k[:, :, a:b], v[:, :, a:b], scale=0.4)
             for a, b in ((0, 10), (10, 25), (25, 40))]
    empty = (np.zeros_like(o), np.full(lse.shape, -np.inf))
    om, lm = oracle.merge_partials(parts + [empty])
    assert np.allclose(om, o, atol=1e-13, rtol=0)
    assert np.allclose(lm, lse, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- closed forms

def test_single_key():
    r = _rng(6)
    q = r.normal(size=(1, 1, 5, 4))
    k = r.normal(size=(1, 1, 1, 4))
    v = r.normal(size=(1, 1, 1, 3))
    o, lse = oracle.attention_forward(q, k, v, scale=0.3)
    assert np.allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (5, 3)), atol=1e-15)
    assert np.allclose(lse[0, 0], 0.3 * (q[0, 0] @ k[0, 0, 0]), atol=1e-14)


def test_equal_scores_give_mean():
    r = _rng(7)
    nk = 13
    q = np.zeros((1, 1, 3, 4))
    k = r.normal(size=(1, 1, nk, 4))
    v = r.normal(size=(1, 1, nk, 2))
    o, lse = oracle.attention_forward(q, k, v, scale=1.0,
                                      bias=np.full((1, 1, 3, nk), 2.5))
    assert np.allclose(o[0, 0], v[0, 0].mean(axis=0), atol=1e-14)
    assert np.allclose(lse, 2.5 + math.log(nk), atol=1e-14)


def test_causal_first_row_and_last_row():
    r = _rng(8)
    q = r.normal(size=(1, 1, 6, 4))
    k = r.normal(size=(1, 1, 6, 4))
    v = r.normal(size=(1, 1, 6, 3))
    o, lse = oracle.attention_forward(q, k, v, scale=0.5, causal=True)
    assert np.allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.5 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14
    on, ln_ = oracle.attention_forward(q, k, v, scale=0.5)
    assert np.allclose(o[0, 0, -1], on[0, 0, -1], atol=1e-15)
    assert abs(lse[0, 0, -1] - ln_[0, 0, -1]) < 1e-14


def test_causal_bottom_right_alignment():
    # flash-attention, Q10: with fewer queries than keys the last query sees
    # every key; with more queries than keys the first rows see none.
    r = _rng(9)
    k = r.normal(size=(1, 1, 7, 4))
    v = r.normal(size=(1, 1, 7, 2))
    q = r.normal(size=(1, 1, 3, 4))
    o, lse = oracle.attention_forward(q, k, v, scale=1.0, causal=True)
    for i in range(3):
        ref_o, ref_l = oracle.attention_forward(q[:, :, i:i + 1], k[:, :, :5 + i],
                                                v[:, :, :5 + i], scale=1.0)
        assert np.allclose(o[0, 0, i], ref_o[0, 0, 0], atol=1e-15)
        assert abs(lse[0, 0, i] - ref_l[0, 0, 0]) < 1e-14
    q2 = r.normal(size=(1, 1, 10, 4))
    o2, l2 = oracle.attention_forward(q2, k, v, scale=1.0, causal=True)
    assert np.all(o2[0, 0, :3] == 0.0) and np.all(l2[0, 0, :3] == -np.inf)
    assert np.all(np.isfinite(l2[0, 0, 3:]))
    assert np.allclose(o2[0, 0, 3], v[0, 0, 0], atol=1e-15)


def test_one_dominant_key():
    r = _rng(10)
    q = r.normal(size=(1, 1, 4, 8))
    k = r.normal(size=(1, 1, 9, 8))
    v = r.normal(size=(1, 1, 9, 5))
    bias = np.zeros((1, 1, 4, 9))
    bias[0, 0, np.arange(4), [2, 5, 0, 8]] = 1e3
    o, _ = oracle.attention_forward(q, k, v, scale=0.1, bias=bias)
    assert np.allclose(o[0, 0], v[0, 0, [2, 5, 0, 8]], atol=1e-12)


# ---------------------------------------------------------------- masks

def test_kv_len_masks():
    r = _rng(11)
    q = r.normal(size=(3, 2, 5, 4))
    k = r.normal(size=(3, 2, 12, 4))
    v = r.normal(size=(3, 2, 12, 3))
    lens = np.array([12, 7, 0])
    o, lse = oracle.attention_forward(q, k, v, scale=0.5, kv_len=lens)
    full_o, full_l = oracle.attention_forward(q, k, v, scale=0.5)
    assert np.array_equal(o[0], full_o[0]) and np.array_equal(lse[0], full_l[0])
    # key length 7 equals truncating the keys, and equals a -inf bias
    t_o, t_l = oracle.attention_forward(q[1:2], k[1:2, :, :7], v[1:2, :, :7],
                                        scale=0.5)
    assert np.allclose(o[1], t_o[0], atol=1e-15)
    assert np.allclose(lse[1], t_l[0], atol=1e-14)
    bias = np.zeros((1, 1, 5, 12))
    bias[..., 7:] = -np.inf
    b_o, b_l = oracle.attention_forward(q[1:2], k[1:2], v[1:2], scale=0.5,
                                        bias=bias)
    assert np.array_equal(b_o[0], o[1]) and np.array_equal(b_l[0], lse[1])
    s = oracle.score_matrix(q[1, 0], k[1, 0], 0.5, valid_keys=7)
    p, _, _ = oracle.masked_softmax(s)
    assert np.all(p[:, 7:] == 0.0)
    # length 0: every key hidden -> zeros and -inf, never NaN
    assert np.all(o[2] == 0.0) and np.all(lse[2] == -np.inf)
    assert not np.isnan(o).any()


def test_rows_subset_matches_full():
    r = _rng(12)
    q = r.normal(size=(2, 3, 20, 8))
    k = r.normal(size=(2, 3, 26, 8))
    v = r.normal(size=(2, 3, 26, 4))
    bias = r.normal(size=(1, 3, 20, 26))
    lens = np.array([26, 9])
    o, lse = oracle.attention_forward(q, k, v, scale=0.3, bias=bias,
                                      kv_len=lens, causal=True)
    rows = [(0, 0, 0), (1, 2, 19), (0, 1, 7), (1, 0, 3), (1, 0, 4)]
    ro, rl = oracle.attention_rows(q, k, v, rows, scale=0.3, bias=bias,
                                   kv_len=lens, causal=True)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(ro[n], o[b, h, i], atol=1e-15)
        assert rl[n] == lse[b, h, i] or abs(rl[n] - lse[b, h, i]) < 1e-14


# ---------------------------------------------------------------- independent evaluations

def test_decimal_50_digits():
    """The definition evaluated in 50-digit decimal arithmetic (no numpy, no
    max subtraction); the oracle must agree to 1e-13."""
    getcontext().prec = 50
    r = _rng(13)
    nq, nk, d, dv = 3, 5, 4, 3
    q = r.normal(size=(nq, d))
    k = r.normal(size=(nk, d))
    v = r.normal(size=(nk, dv))
    bias = r.normal(size=(nq, nk))
    scale = 0.37
    o, lse = oracle.attention_forward(q[None, None], k[None, None], v[None, None],
                                      scale=scale, bias=bias[None, None])
    D = Decimal
    for i in range(nq):
        sc = []
        for j in range(nk):
            dot = sum(D(float(q[i, t])) * D(float(k[j, t])) for t in range(d))
            sc.append(D(scale) * dot + D(float(bias[i, j])))
        ex = [x.exp() for x in sc]
        tot = sum(ex)
        for c in range(dv):
            want = sum(ex[j] * D(float(v[j, c])) for j in range(nk)) / tot
            assert abs(float(want) - o[0, 0, i, c]) < 1e-13
        assert abs(float(tot.ln()) - lse[0, 0, i]) < 1e-13


def test_brute_force_loops():
    """Plain loops with exp(s) / sum exp(s) (no max subtraction) on tiny
    inputs with a bias, causal masking and a key length."""
    r = _rng(14)
    B, H, nq, nk, d, dv = 2, 2, 4, 6, 3, 2
    q = r.normal(size=(B, H, nq, d))
    k = r.normal(size=(B, H, nk, d))
    v = r.normal(size=(B, H, nk, dv))
    bias = r.normal(size=(B, 1, nq, nk))
    lens = [6, 4]
    scale = 0.8
    o, lse = oracle.attention_forward(q, k, v, scale=scale, bias=bias,
                                      kv_len=lens, causal=True)
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                w = []
                for j in range(nk):
                    ok = j < lens[b] and j <= i + (nk - nq)
                    if ok:
                        s = scale * sum(q[b, h, i, t] * k[b, h, j, t] for t in range(d))
                        w.append(math.exp(s + bias[b, 0, i, j]))
                    else:
                        w.append(0.0)
                tot = sum(w)
                assert abs(math.log(tot) - lse[b, h, i]) < 1e-13
                for c in range(dv):
                    want = sum(w[j] * v[b, h, j, c] for j in range(nk)) / tot
                    assert abs(want - o[b, h, i, c]) < 1e-14


def test_layout_is_batch_head_seq_dim():
    # A [B, H, N, d] input whose H and N are swapped must give a different
    # answer: the oracle attends over axis 2.
    r = _rng(15)
    q = r.normal(size=(1, 3, 5, 4))
    k = r.normal(size=(1, 3, 5, 4))
    v = r.normal(size=(1, 3, 5, 4))
    o, _ = oracle.attention_forward(q, k, v, scale=0.5)
    for h in range(3):
        oh, _ = oracle.attention_forward(q[:, h:h + 1], k[:, h:h + 1],
                                         v[:, h:h + 1], scale=0.5)
        assert np.allclose(o[:, h], oh[:, 0], atol=1e-15)
    ot, _ = oracle.attention_forward(q.transpose(0, 2, 1, 3), k.transpose(0, 2, 1, 3),
                                     v.transpose(0, 2, 1, 3), scale=0.5)
    assert not np.allclose(ot.transpose(0, 2, 1, 3), o, atol=1e-3)


# ----------------------------------------------------------- sliding window
# The kept key sets below are listed by hand from the reading of the pages'
# window (left, right) around the bottom-right-aligned diagonal i + Nk - Nq,
# not computed by the oracle's formula.
WINDOW_CASES = [
    # (Nq, Nk, window, kept keys of each query row)
    (6, 6, (2, 0), [[0], [0, 1], [0, 1, 2], [1, 2, 3], [2, 3, 4], [3, 4, 5]]),
    (3, 7, (1, 1), [[3, 4, 5], [4, 5, 6], [5, 6]]),
    (5, 5, (2, -1), [[0, 1, 2, 3, 4], [0, 1, 2, 3, 4], [0, 1, 2, 3, 4], [1, 2, 3, 4],
                     [2, 3, 4]]),
    (4, 4, (-1, 1), [[0, 1], [0, 1, 2], [0, 1, 2, 3], [0, 1, 2, 3]]),
    (5, 3, (0, 1), [[], [0], [0, 1], [1, 2], [2]]),
    (2, 6, (0, 0), [[4], [5]]),
]


def test_window_kept_keys():
    for nq, nk, window, kept in WINDOW_CASES:
        _check_window_case(nq, nk, window, kept)


def _check_window_case(nq, nk, window, kept):
    # Uniform scores (q = 0): each row's output is the mean of the values of
    # its kept keys and its LSE is ln(count); a row with none is 0 / -inf.
    r = _rng(30 + nq * nk)
    q = np.zeros((1, 1, nq, 4))
    k = r.normal(size=(1, 1, nk, 4))
    v = r.normal(size=(1, 1, nk, 3))
    o, lse = oracle.attention_forward(q, k, v, scale=1.0, window=window)
    for i, keys in enumerate(kept):
        if keys:
            assert np.allclose(o[0, 0, i], v[0, 0, keys].mean(axis=0), atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(len(keys))) < 1e-14
        else:
            assert np.all(o[0, 0, i] == 0.0) and lse[0, 0, i] == -np.inf
    # random queries: each row equals plain attention over its kept keys only
    q = r.normal(size=(1, 1, nq, 4))
    o, lse = oracle.attention_forward(q, k, v, scale=0.7, window=window)
    for i, keys in enumerate(kept):
        if not keys:
            continue
        ro, rl = oracle.attention_forward(q[:, :, i:i + 1], k[:, :, keys], v[:, :, keys],
                                          scale=0.7)
        assert np.allclose(o[0, 0, i], ro[0, 0, 0], atol=1e-14)
        assert abs(lse[0, 0, i] - rl[0, 0, 0]) < 1e-13


def test_window_special_cases():
    r = _rng(40)
    q = r.normal(size=(2, 2, 9, 4))
    k = r.normal(size=(2, 2, 11, 4))
    v = r.normal(size=(2, 2, 11, 3))
    plain = oracle.attention_forward(q, k, v, scale=0.5)
    causal = oracle.attention_forward(q, k, v, scale=0.5, causal=True)
    for w in [(-1, -1), (None, None), (11, 11), (100, 9)]:
        o, lse = oracle.attention_forward(q, k, v, scale=0.5, window=w)
        assert np.array_equal(o, plain[0]) and np.array_equal(lse, plain[1])
    for w in [(-1, 0), (20, 0)]:
        o, lse = oracle.attention_forward(q, k, v, scale=0.5, window=w)
        assert np.array_equal(o, causal[0]) and np.array_equal(lse, causal[1])
    # causal and a right bound: the causal side wins
    o, lse = oracle.attention_forward(q, k, v, scale=0.5, causal=True, window=(-1, 3))
    assert np.array_equal(o, causal[0])


# ------------------------------------------------------- packed sequences
def _varlen_case(seed, lens_q, lens_k, H=3, Hk=3, d=4):
    r = _rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    q = r.normal(size=(int(cu_q[-1]), H, d))
    k = r.normal(size=(int(cu_k[-1]), Hk, d))
    v = r.normal(size=(int(cu_k[-1]), Hk, 2))
    return q, k, v, cu_q, cu_k


def test_varlen_equals_padded_batch_with_key_lengths():
    # Another route to the same rows: pad every sequence to the longest, mask
    # the padded keys with kv_len, and read back the real rows only.
    lens = [5, 1, 7, 0, 3]
    q, k, v, cu_q, cu_k = _varlen_case(50, lens, lens)
    L = max(lens)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.6, causal=causal)
        qp = np.zeros((len(lens), 3, L, 4))
        kp = np.zeros((len(lens), 3, L, 4))
        vp = np.zeros((len(lens), 3, L, 2))
        for s, n in enumerate(lens):
            qp[s, :, :n] = q[cu_q[s]:cu_q[s + 1]].transpose(1, 0, 2)
            kp[s, :, :n] = k[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)
            vp[s, :, :n] = v[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)
        po, pl = oracle.attention_forward(qp, kp, vp, scale=0.6, kv_len=lens, causal=causal)
        for s, n in enumerate(lens):
            for i in range(n):
                row = cu_q[s] + i
                assert np.allclose(o[row], po[s, :, i], atol=1e-14)
                assert np.allclose(lse[:, row], pl[s, :, i], atol=1e-14)


def test_varlen_single_sequence_and_unequal_lengths():
    # one sequence covering the packed tensors is the plain forward; with
    # fewer query rows than keys each sequence keeps its own bottom-right
    # causal alignment (its last query sees all of its keys)
    q, k, v, cu_q, cu_k = _varlen_case(51, [6], [6])
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.4, causal=True)
    ro, rl = oracle.attention_forward(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None],
                                      v.transpose(1, 0, 2)[None], scale=0.4, causal=True)
    assert np.allclose(o, ro[0].transpose(1, 0, 2), atol=1e-15)
    assert np.allclose(lse, rl[0], atol=1e-15)
    q, k, v, cu_q, cu_k = _varlen_case(52, [2, 3], [4, 6])
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.4, causal=True)
    for s in range(2):
        last = cu_q[s + 1] - 1
        ro, rl = oracle.attention_forward(q[last:last + 1].transpose(1, 0, 2)[None],
                                          k[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)[None],
                                          v[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)[None],
                                          scale=0.4)
        assert np.allclose(o[last], ro[0, :, 0], atol=1e-14)
    # a sequence with no keys: zero rows, -inf LSE
    q, k, v, cu_q, cu_k = _varlen_case(53, [2, 2], [3, 0])
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=1.0)
    assert np.all(o[2:] == 0.0) and np.all(lse[:, 2:] == -np.inf)


def test_varlen_grouped_heads():
    # query head h reads key/value head h // (H / Hk): with Hk = 1 every
    # query head of a sequence sees the same keys
    q, k, v, cu_q, cu_k = _varlen_case(54, [3, 4], [5, 2], H=4, Hk=1)
    o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale=0.5)
    for s in range(2):
        for h in range(4):
            ro, rl = oracle.attention_forward(
                q[cu_q[s]:cu_q[s + 1], h][None, None], k[cu_k[s]:cu_k[s + 1], 0][None, None],
                v[cu_k[s]:cu_k[s + 1], 0][None, None], scale=0.5)
            assert np.allclose(o[cu_q[s]:cu_q[s + 1], h], ro[0, 0], atol=1e-14)


# ----------------------------------------------------------------- backward
def _loss(q, k, v, do, **kw):
    # L = sum(O o dO): its gradient with respect to O is dO
    o, _ = oracle.attention_forward(q, k, v, **kw)
    return float((o * do).sum())


def _finite_difference(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + eps
        up = f()
        x[idx] = old - eps
        dn = f()
        x[idx] = old
        g[idx] = (up - dn) / (2 * eps)
    return g


def test_backward_matches_finite_differences():
    # central differences of L = sum(O o dO) on tiny inputs: an independent
    # route to the gradients (no softmax Jacobian written anywhere)
    r = _rng(70)
    cases = [dict(causal=False), dict(causal=True),
             dict(bias=r.normal(size=(1, 2, 4, 5)) * 0.5, kv_len=[4, 3]),
             dict(window=(1, 1)), dict(causal=True, window=(2, 0))]
    for nq, nk in ((4, 5), (4, 4)):          # a square case too (a transposed P is square)
        for kw in cases:
            if nk == 4 and "bias" in kw:
                continue
            q = r.normal(size=(2, 2, nq, 3))
            k = r.normal(size=(2, 2, nk, 3))
            v = r.normal(size=(2, 2, nk, 3))
            do = r.normal(size=(2, 2, nq, 3))
            dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.7, **kw)
            for x, g in ((q, dq), (k, dk), (v, dv)):
                fd = _finite_difference(lambda: _loss(q, k, v, do, scale=0.7, **kw), x)
                assert np.allclose(g, fd, atol=1e-7), kw


def test_backward_grouped_heads_sum_over_the_group():
    # with Hk = 1 the key/value gradient is the sum over the query heads
    r = _rng(71)
    q = r.normal(size=(1, 3, 4, 2))
    k = r.normal(size=(1, 1, 6, 2))
    v = r.normal(size=(1, 1, 6, 2))
    do = r.normal(size=(1, 3, 4, 2))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.5, causal=True)
    fd_k = _finite_difference(lambda: _loss_gqa(q, k, v, do), k)
    assert np.allclose(dk, fd_k, atol=1e-7)
    fd_v = _finite_difference(lambda: _loss_gqa(q, k, v, do), v)
    assert np.allclose(dv, fd_v, atol=1e-7)


def _loss_gqa(q, k, v, do):
    kx = np.repeat(k, q.shape[1] // k.shape[1], axis=1)
    vx = np.repeat(v, q.shape[1] // v.shape[1], axis=1)
    return _loss(q, kx, vx, do, scale=0.5, causal=True)


def test_backward_identities():
    # D = rowsum(dO o O) = rowsum(dP o P) (the pages' identity), dS sums to
    # zero along each row, a fully masked row has zero dQ, keys past kv_len
    # get zero dK and dV, and a uniform shift of dO along V's row space does
    # not change dQ / dK (softmax is invariant to it)
    r = _rng(72)
    q = r.normal(size=(1, 2, 5, 3))
    k = r.normal(size=(1, 2, 7, 3))
    v = r.normal(size=(1, 2, 7, 3))
    do = r.normal(size=(1, 2, 5, 3))
    o, _ = oracle.attention_forward(q, k, v, scale=0.9)
    s = 0.9 * q[0, 0] @ k[0, 0].T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    assert np.allclose((do[0, 0] * o[0, 0]).sum(axis=1), (p * dp).sum(axis=1), atol=1e-14)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale=0.9, kv_len=[4])
    assert np.all(dk[0, :, 4:] == 0.0) and np.all(dv[0, :, 4:] == 0.0)
    q2 = r.normal(size=(1, 1, 6, 3))
    dq2, _, _ = oracle.attention_backward(q2, k[:, :1, :4], v[:, :1, :4], r.normal(size=(1, 1, 6, 3)),
                                          scale=1.0, causal=True)
    assert np.all(dq2[0, 0, :2] == 0.0)          # rows 0, 1 see no key (Nq > Nk)
    c = r.normal(size=(3,))
    base = oracle.attention_backward(q, k, v, do, scale=0.9)
    shifted = oracle.attention_backward(q, k, v + c, do, scale=0.9)
    assert np.allclose(base[0], shifted[0], atol=1e-13)
    assert np.allclose(base[1], shifted[1], atol=1e-13)
