"""Plain float64 attention, written from the definition.

TEST INFRASTRUCTURE (see the package docstring): nothing on the product path
imports this module.

Conventions (the readings of the pages this file takes):

* Layout [B, H, N, d], the PyTorch order; the pages warn that the other common
  order [B, N, H, d] silently attends over the wrong axis if mixed up
  [flash-attention (stanleyjacob.dev), Part II, on the layout].
* ``scale`` multiplies Q K^T only; the additive bias is added after it,
  unscaled [Understanding FlashAttention Pt 1, §0.2 "Notation": S = QK^T/sqrt(d) + B].
* Masked positions get score -inf and therefore probability exactly 0
  [same page, §2.4 on masks applied before the exponentials, and §3.5].
* Causal masking is aligned to the bottom-right corner of the score matrix:
  key j is hidden from query i when j > i + (Nk - Nq) [flash-attention,
  Q10 on unequal query/key lengths]. With Nq == Nk this is "j > i".
* ``kv_len[b]`` hides keys j >= kv_len[b] of batch entry b, the same as an
  additive -inf bias on the padded keys.
* A sliding window (left, right) keeps key j for query i only when
  i + (Nk - Nq) - left <= j <= i + (Nk - Nq) + right, a band around the same
  bottom-right-aligned diagonal; a negative (or None) bound leaves that side
  open, and causal masking is the band with right = 0 and no left bound. The
  pages name the window (left and right sizes, -1 for "no window") and the
  band of tiles it leaves, but print no formula; this is the plainest reading
  that agrees with their causal alignment [Understanding FlashAttention Pt 1,
  §3.5, connection to local attention; FlashAttention, Explained, §14;
  flash-attention, Part III and Lab 3, window_size_left/right].
* A row whose scores are all -inf yields O = 0 and LSE = -inf (log of a zero
  denominator) instead of NaN [flash-attention, Part VI, fully masked rows].
* LSE is the natural logarithm of the row's denominator, in the units of the
  scaled + biased scores: LSE_i = m_i + ln l_i [flash-attention, Part VI].
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def score_matrix(qh, kh, scale, bias=None, valid_keys=None, causal=False,
                 q_positions=None, n_q=None, window=None) -> np.ndarray:
    """Scores of one head: S = scale * Q K^T + B, then the masks as -inf.

    qh: [nq, d] queries (rows of Q), kh: [Nk, d] keys.
    bias: None or an array broadcastable to [nq, Nk], added unscaled.
    valid_keys: None or an integer; keys j >= valid_keys are masked.
    causal: mask key j for query i when j > i + (Nk - n_q).
    q_positions: absolute query index of each row of ``qh`` (default 0..nq-1);
      n_q: the full query length Nq that the causal alignment uses
      (default nq). These two let a caller evaluate a subset of rows.
    window: None or (left, right); key j is kept for query i only when
      i + (Nk - n_q) - left <= j <= i + (Nk - n_q) + right (None or a
      negative bound: that side open).

    [Understanding FlashAttention Pt 1, §0.2 "Notation" for S;
     §3.5 "Causal Masking and Tile Skipping" for the causal pattern.]
    """
    qh = _f64(qh)
    kh = _f64(kh)
    nq, nk = qh.shape[0], kh.shape[0]
    s = float(scale) * (qh @ kh.T)
    if bias is not None:
        s = s + np.broadcast_to(_f64(bias), (nq, nk))
    if q_positions is None:
        q_positions = np.arange(nq)
    q_positions = np.asarray(q_positions, dtype=np.int64)
    if n_q is None:
        n_q = nq
    j = np.arange(nk, dtype=np.int64)
    hide = np.zeros((nq, nk), dtype=bool)
    if valid_keys is not None:
        hide |= (j >= int(valid_keys))[None, :]
    diag = q_positions[:, None] + (nk - int(n_q))   # the aligned diagonal
    if causal:
        hide |= j[None, :] > diag
    if window is not None:
        left, right = window
        if left is not None and left >= 0:
            hide |= j[None, :] < diag - int(left)
        if right is not None and right >= 0:
            hide |= j[None, :] > diag + int(right)
    if hide.any():
        s = np.where(hide, -np.inf, s)
    return s


def masked_softmax(s) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row softmax with the max subtracted first (the "safe" softmax).

    Returns (P, m, l): P = exp(S - m) / l with m the row maximum and l the
    row sum of exp(S - m). A row that is entirely -inf, or has no keys at
    all, gets P = 0, m = -inf, l = 0 rather than NaN.

    [Understanding FlashAttention Pt 1, §2.2 "Softmax Is the Difficult Part of
     Streaming"; FlashAttention, Explained, §9.]
    """
    s = _f64(s)
    if s.shape[-1] == 0:                      # no keys at all: an empty row
        z = np.zeros(s.shape[:-1])
        return np.zeros(s.shape), np.full(s.shape[:-1], -np.inf), z
    m = s.max(axis=-1)
    dead = ~np.isfinite(m) & (m < 0)          # m == -inf: every key masked
    m_ref = np.where(dead, 0.0, m)
    e = np.exp(s - m_ref[..., None])          # exp(-inf) == 0 exactly
    l = e.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(dead[..., None], 0.0, e / l[..., None])
    return p, m, l


def _head_forward(qh, kh, vh, scale, bias, valid_keys, causal, q_positions, n_q,
                  window=None):
    s = score_matrix(qh, kh, scale, bias, valid_keys, causal, q_positions, n_q, window)
    p, m, l = masked_softmax(s)
    o = p @ _f64(vh)
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def _bias_for(bias, b, h):
    if bias is None:
        return None
    bias = _f64(bias)
    if bias.ndim != 4:
        raise ValueError("bias must be 4-D [B|1, H|1, Nq, Nk]")
    return bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]


def attention_forward(q, k, v, *, scale, bias=None, kv_len=None, causal=False,
                      window=None):
    """O = softmax_row(scale * Q K^T + B) V and LSE, for [B, H, N, d] inputs.

    q: [B, H, Nq, d], k: [B, H, Nk, d], v: [B, H, Nk, dv] (any real dtype;
    widened to float64). bias: None or [B|1, H|1, Nq, Nk]. kv_len: None or
    B integers. window: None or (left, right), see ``score_matrix``.
    Returns (O [B, H, Nq, dv], LSE [B, H, Nq]) in float64.

    Each head materialises its full S and P, exactly the three-pass standard
    algorithm the fused kernel replaces [Understanding FlashAttention Pt 1,
    §0.1; FlashAttention: Mathematical Foundations..., §1].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, _ = q.shape
    dv = v.shape[3]
    o = np.zeros((B, H, Nq, dv))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        vk = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            o[b, h], lse[b, h] = _head_forward(
                q[b, h], k[b, h], v[b, h], scale, _bias_for(bias, b, h), vk,
                causal, None, Nq, window)
    return o, lse


def attention_rows(q, k, v, rows: Iterable[Sequence[int]], *, scale, bias=None,
                   kv_len=None, causal=False, window=None):
    """The same function as ``attention_forward`` for selected rows only.

    rows: iterable of (b, h, i). Returns (O [n, dv], LSE [n]) in row order.
    Used to check outputs of shapes too large to evaluate in full; each row
    still sees every key of its head.
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    Nq = q.shape[2]
    # group by head so each head's keys are widened once
    by_head: dict[tuple[int, int], list[tuple[int, int]]] = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    o = np.zeros((len(rows), v.shape[3]))
    lse = np.zeros(len(rows))
    for (b, h), items in by_head.items():
        idx = np.array([i for _, i in items], dtype=np.int64)
        bh = _bias_for(bias, b, h)
        bsel = None if bh is None else bh[idx]
        vk = None if kv_len is None else int(kv_len[b])
        oh, lh = _head_forward(_f64(q[b, h][idx]), _f64(k[b, h]), _f64(v[b, h]),
                               scale, bsel, vk, causal, idx, Nq, window)
        for r, (n, _) in enumerate(items):
            o[n] = oh[r]
            lse[n] = lh[r]
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, *, scale, causal=False, window=None):
    """The forward over packed variable-length sequences.

    q: [Tq, H, d], k: [Tk, Hk, d], v: [Tk, Hk, dv] (token-major packing);
    cu_q, cu_k: num_seqs + 1 cumulative offsets. Sequence s is plain
    attention (``attention_forward``, with its causal alignment and window)
    of rows q[cu_q[s]:cu_q[s+1]] against keys k[cu_k[s]:cu_k[s+1]]; query
    head h reads key/value head h // (H / Hk). Returns (O [Tq, H, dv],
    LSE [H, Tq]); rows outside every sequence are NaN.
    [flash-attention (stanleyjacob.dev), Part II, variable-length batches
     and grouped-query attention.]
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, H, _ = q.shape
    rep = H // k.shape[1]
    o = np.full((Tq, H, v.shape[2]), np.nan)
    lse = np.full((H, Tq), np.nan)
    for s in range(len(cu_q) - 1):
        a0, a1 = int(cu_q[s]), int(cu_q[s + 1])
        c0, c1 = int(cu_k[s]), int(cu_k[s + 1])
        if a1 <= a0:
            continue
        qs = q[a0:a1].transpose(1, 0, 2)[None]                      # [1, H, n, d]
        ks = np.repeat(k[c0:c1].transpose(1, 0, 2), rep, axis=0)[None]
        vs = np.repeat(v[c0:c1].transpose(1, 0, 2), rep, axis=0)[None]
        os_, ls_ = attention_forward(qs, ks, vs, scale=scale, causal=causal, window=window)
        o[a0:a1] = os_[0].transpose(1, 0, 2)
        lse[:, a0:a1] = ls_[0]
    return o, lse


def attention_backward(q, k, v, do, *, scale, bias=None, kv_len=None, causal=False,
                       window=None):
    """Gradients of the forward with respect to Q, K and V, in float64.

    For an upstream gradient dO of O = P V with P = softmax_row(S),
    S = scale * Q K^T + B (masks as -inf):
        dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij,
        dS = P o (dP - D[:, None]),   dQ = scale * dS K,   dK = scale * dS^T Q.
    A masked pair has P_ij = 0 and therefore dS_ij = 0; a row with no
    visible key contributes nothing. q, do: [B, H, Nq, d], k, v: [B, Hk,
    Nk, d] with query head h reading key/value head h // (H / Hk); dK and dV
    of a key/value head sum over the query heads that read it. The bias is a
    constant here (no gradient is returned for it).
    Returns (dQ, dK, dV) with the shapes of q, k, v.
    [Understanding FlashAttention Pt 1, §3.6; FlashAttention, Explained,
     §17; FlashAttention: Mathematical Foundations..., §4.]
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, _ = q.shape
    Hk = k.shape[1]
    rep = H // Hk
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        vk = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            hk = h // rep
            s = score_matrix(q[b, h], k[b, hk], scale, _bias_for(bias, b, h), vk, causal,
                             None, Nq, window)
            p, _, _ = masked_softmax(s)
            dvh = p.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            dd = (p * dp).sum(axis=1)
            ds = p * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h])
            dv[b, hk] += dvh
    return dq, dk, dv


def online_softmax_scalar(scores, values):
    """One query row, one key at a time: the online normaliser with a value
    accumulator.

    Starting from m = -inf, l = 0, a = 0, each score x_j updates
        m_j = max(m_{j-1}, x_j)
        l_j = l_{j-1} exp(m_{j-1} - m_j) + exp(x_j - m_j)
        a_j = a_{j-1} exp(m_{j-1} - m_j) + exp(x_j - m_j) v_j
    and the output is a / l [Understanding FlashAttention Pt 1, §2.3
    "Online Softmax from First Principles"]. A -inf score contributes nothing;
    while the running maximum is still -inf the old state is empty and is
    kept at zero. Returns (o, lse, m, l).
    """
    scores = _f64(scores).ravel()
    values = _f64(values).reshape(len(scores), -1)
    m, l = -math.inf, 0.0
    a = np.zeros(values.shape[1])
    for x, vj in zip(scores, values):
        m_new = max(m, x)
        if m_new == -math.inf:
            continue
        alpha = math.exp(m - m_new)        # exp(-inf) = 0 for the empty state
        w = math.exp(x - m_new)
        l = l * alpha + w
        a = a * alpha + w * vj
        m = m_new
    if l == 0.0:
        return np.zeros_like(a), -math.inf, m, l
    return a / l, m + math.log(l), m, l


def online_softmax_blocked(scores, values, block):
    """The blockwise merge recurrence over the keys, for one query row or a
    block of query rows.

    scores: [n] (one row) or [r, n] (r rows sharing the values; masked
    positions are -inf and contribute zero probability); values: [n, dv].
    The state of each row is (m, l, a): the largest score so far, the sum of
    exp(score - m) so far and the unnormalised value accumulator. Each block
    of `block` consecutive keys, with scores s and values V_b, applies
        m_b = max(s),  m' = max(m, m_b),  alpha = exp(m - m'),  p = exp(s - m'),
        l' = alpha l + sum(p),  a' = alpha a + p^T V_b,  (m, l, a) <- (m', l', a')
    row by row, and at the end o = a / l [Understanding FlashAttention Pt 1,
    §2.4 "The Blockwise Merge Recurrence", including its closing remarks on
    blocks of query rows (m and l row vectors, a a matrix) and on masks
    applied before the exponentials]. A row whose maximum is still -inf after
    a block (nothing visible yet) keeps its empty state. Returns
    (o, lse, m, l); o = 0 and lse = -inf for a row that saw no key.
    """
    sc = _f64(scores)
    one_row = sc.ndim == 1
    sc = sc.reshape(1, -1) if one_row else sc.reshape(-1, sc.shape[-1])
    n_rows, n = sc.shape
    vals = _f64(values).reshape(n, -1)
    width = int(block)
    if width < 1:
        raise ValueError("block must be >= 1")
    m = np.full(n_rows, -np.inf)            # running maximum per row
    ell = np.zeros(n_rows)                  # running denominator per row
    acc = np.zeros((n_rows, vals.shape[1]))  # running accumulator per row
    for lo in range(0, n, width):
        s_blk = sc[:, lo:lo + width]
        v_blk = vals[lo:lo + width]
        m_blk = s_blk.max(axis=1)
        m_next = np.maximum(m, m_blk)
        live = np.isfinite(m_next)           # rows that have seen a key
        ref = np.where(live, m_next, 0.0)    # any finite stand-in for dead rows
        alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
        p = np.where(live[:, None], np.exp(s_blk - ref[:, None]), 0.0)
        ell = np.where(live, alpha * ell + p.sum(axis=1), ell)
        acc = np.where(live[:, None], alpha[:, None] * acc + p @ v_blk, acc)
        m = np.where(live, m_next, m)
    seen = ell > 0.0
    safe = np.where(seen, ell, 1.0)
    o = np.where(seen[:, None], acc / safe[:, None], 0.0)
    lse = np.where(seen, m + np.log(safe), -np.inf)
    if one_row:
        return o[0], float(lse[0]), float(m[0]), float(ell[0])
    return o, lse, m, ell


def merge_partials(parts):
    """Combine partial (o_k, lse_k) results over disjoint key sets.

    With m = max_k lse_k, the weights are w_k = exp(lse_k - m) and
    o = sum_k w_k o_k / sum_k w_k, lse = m + ln(sum_k w_k). This is the
    combination of partial attention results by their log-sum-exps
    [FlashAttention: Mathematical Foundations..., §7 on Flash-Decoding;
     flash-attention (stanleyjacob.dev), Part VI and Q12], written with the
    LSE in place of the pair (m_k, l_k) since lse_k = m_k + ln l_k.
    parts: sequence of (o [..., dv], lse [...]). Rows whose parts are all
    -inf give o = 0, lse = -inf.
    """
    os_ = [_f64(o) for o, _ in parts]
    ls_ = [_f64(l) for _, l in parts]
    m = np.max(np.stack(ls_), axis=0)
    dead = ~np.isfinite(m) & (m < 0)
    m_ref = np.where(dead, 0.0, m)
    w = [np.exp(l - m_ref) for l in ls_]
    tot = np.sum(np.stack(w), axis=0)
    num = sum(wk[..., None] * ok for wk, ok in zip(w, os_))
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(dead[..., None], 0.0, num / tot[..., None])
        lse = np.where(dead, -np.inf, m_ref + np.log(np.where(dead, 1.0, tot)))
    return o, lse
