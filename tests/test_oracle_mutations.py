"""Plant plausible mistakes in the CPU oracle and check the pins catch each.

Every mutation replaces one oracle function with a copy that has one slip
(a dropped term, a wrong sign or index, a transposed operand, a wrong log
base...). The pin tests of test_oracle_pins.py are then run against the
mutated oracle; at least one of them must fail. Nothing here touches a GPU.
"""

import inspect
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import test_oracle_pins as pins

_orig = {name: getattr(oa, name) for name in (
    "score_matrix", "masked_softmax", "_head_forward", "online_softmax_blocked",
    "online_softmax_scalar", "merge_partials", "attention_varlen", "attention_backward")}


def _scores(variant):
    def score_matrix(qh, kh, scale, bias=None, valid_keys=None, causal=False,
                     q_positions=None, n_q=None, window=None):
        qh = np.asarray(qh, dtype=np.float64)
        kh = np.asarray(kh, dtype=np.float64)
        nq, nk = qh.shape[0], kh.shape[0]
        raw = qh @ kh.T
        if variant == "scale_squared":
            s = scale * scale * raw
        else:
            s = scale * raw
        if bias is not None and variant != "drop_bias":
            b = np.broadcast_to(np.asarray(bias, dtype=np.float64), (nq, nk))
            s = s + (scale * b if variant == "bias_scaled" else b)
        qp = np.arange(nq) if q_positions is None else np.asarray(q_positions)
        n_q = nq if n_q is None else n_q
        j = np.arange(nk)
        hide = np.zeros((nq, nk), dtype=bool)
        if valid_keys is not None:
            if variant == "kv_len_off_by_one":
                hide |= (j > int(valid_keys))[None, :]
            else:
                hide |= (j >= int(valid_keys))[None, :]
        if causal:
            if variant == "causal_top_left":
                hide |= j[None, :] > qp[:, None]
            elif variant == "causal_diag_masked":
                hide |= j[None, :] >= qp[:, None] + (nk - int(n_q))
            else:
                hide |= j[None, :] > qp[:, None] + (nk - int(n_q))
        if window is not None:
            left, right = window
            diag = qp[:, None] + (0 if variant == "window_top_left" else nk - int(n_q))
            if variant == "window_sides_swapped":
                left, right = right, left
            if left is not None and left >= 0:
                if variant == "window_left_exclusive":
                    hide |= j[None, :] <= diag - int(left)
                else:
                    hide |= j[None, :] < diag - int(left)
            if right is not None and right >= 0 and variant != "window_drop_right":
                hide |= j[None, :] > diag + int(right)
        return np.where(hide, -np.inf, s)
    return score_matrix


def _softmax(variant):
    def masked_softmax(s):
        s = np.asarray(s, dtype=np.float64)
        m = s.max(axis=-1)
        dead = ~np.isfinite(m) & (m < 0)
        m_ref = m if variant == "no_dead_row_guard" else np.where(dead, 0.0, m)
        if variant == "sign_flip":
            e = np.exp(m_ref[..., None] - s)
            e = np.where(np.isfinite(s), e, 0.0)
        else:
            e = np.exp(s - m_ref[..., None])
        l = e.sum(axis=-1)
        with np.errstate(invalid="ignore", divide="ignore"):
            if variant == "no_dead_row_guard":
                p = e / l[..., None]
            else:
                p = np.where(dead[..., None], 0.0, e / l[..., None])
        return p, m, l
    return masked_softmax


def _head(variant):
    def _head_forward(qh, kh, vh, scale, bias, valid_keys, causal, q_positions, n_q,
                      window=None):
        s = oa.score_matrix(qh, kh, scale, bias, valid_keys, causal, q_positions, n_q, window)
        p, m, l = oa.masked_softmax(s)
        vh = np.asarray(vh, dtype=np.float64)
        if variant == "pv_transposed" and p.shape[0] == p.shape[1]:
            o = p.T @ vh
        else:
            o = p @ vh
        with np.errstate(divide="ignore"):
            safe = np.where(l > 0, l, 1.0)
            if variant == "lse_log2":
                core = m + np.log2(safe)
            elif variant == "lse_drops_max":
                core = np.log(safe)
            else:
                core = m + np.log(safe)
            lse = np.where(l > 0, core, -np.inf)
        return o, lse
    return _head_forward


def _blocked(variant):
    def online_softmax_blocked(scores, values, block):
        sc = np.asarray(scores, dtype=np.float64)
        one_row = sc.ndim == 1
        sc = sc.reshape(1, -1) if one_row else sc.reshape(-1, sc.shape[-1])
        n_rows, n = sc.shape
        vals = np.asarray(values, dtype=np.float64).reshape(n, -1)
        m = np.full(n_rows, -np.inf)
        ell = np.zeros(n_rows)
        acc = np.zeros((n_rows, vals.shape[1]))
        for lo in range(0, n, int(block)):
            s_blk = sc[:, lo:lo + int(block)]
            v_blk = vals[lo:lo + int(block)]
            m_next = np.maximum(m, s_blk.max(axis=1))
            live = np.isfinite(m_next)
            ref = np.where(live, m_next, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
            p = np.where(live[:, None], np.exp(s_blk - ref[:, None]), 0.0)
            a_l = np.ones(n_rows) if variant == "blocked_no_rescale_l" else alpha
            a_a = np.ones(n_rows) if variant == "blocked_no_rescale_a" else alpha
            ell = np.where(live, a_l * ell + p.sum(axis=1), ell)
            acc = np.where(live[:, None], a_a[:, None] * acc + p @ v_blk, acc)
            m = np.where(live, m_next, m)
        seen = ell > 0.0
        safe = np.where(seen, ell, 1.0)
        o = np.where(seen[:, None], acc / safe[:, None], 0.0)
        lse = np.where(seen, m + np.log(safe), -np.inf)
        if one_row:
            return o[0], float(lse[0]), float(m[0]), float(ell[0])
        return o, lse, m, ell
    return online_softmax_blocked


def _scalar(variant):
    def online_softmax_scalar(scores, values):
        scores = np.asarray(scores, dtype=np.float64).ravel()
        values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
        m, l = -math.inf, 0.0
        a = np.zeros(values.shape[1])
        for x, vj in zip(scores, values):
            m_new = max(m, x)
            if m_new == -math.inf:
                continue
            alpha = math.exp(m - m_new)
            w = math.exp(x - m_new)
            l = l * alpha + w
            a = (a if variant == "scalar_no_rescale_a" else a * alpha) + w * vj
            m = m_new
        if l == 0.0:
            return np.zeros_like(a), -math.inf, m, l
        return a / l, m + math.log(l), m, l
    return online_softmax_scalar


def _merge(variant):
    def merge_partials(parts):
        os_ = [np.asarray(o, dtype=np.float64) for o, _ in parts]
        ls_ = [np.asarray(l, dtype=np.float64) for _, l in parts]
        if variant == "merge_plain_mean":
            return sum(os_) / len(os_), np.max(np.stack(ls_), axis=0)
        return _orig["merge_partials"](parts)
    return merge_partials


def _varlen(variant):
    def attention_varlen(q, k, v, cu_q, cu_k, *, scale, causal=False, window=None):
        if variant == "varlen_keys_from_query_offsets":
            return _orig["attention_varlen"](q, k, v, cu_q, cu_q, scale=scale, causal=causal,
                                             window=window)
        if variant == "varlen_keys_of_all_sequences":
            n = len(cu_k) - 1
            whole = np.array([0] + [int(cu_k[-1])] * n)
            starts = np.array([0] * (n + 1))
            o, lse = _orig["attention_varlen"](q, k, v, cu_q, whole, scale=scale,
                                               causal=causal, window=window)
            return o, lse
        return _orig["attention_varlen"](q, k, v, cu_q, cu_k, scale=scale, causal=causal,
                                         window=window)
    return attention_varlen


def _backward(variant):
    def attention_backward(q, k, v, do, *, scale, bias=None, kv_len=None, causal=False,
                           window=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, Nq, _ = q.shape
        rep = H // k.shape[1]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            vk = None if kv_len is None else int(kv_len[b])
            for h in range(H):
                hk = h // rep
                s = oa.score_matrix(q[b, h], k[b, hk], scale, oa._bias_for(bias, b, h), vk,
                                    causal, None, Nq, window)
                p, _, _ = oa.masked_softmax(s)
                dp = do[b, h] @ v[b, hk].T
                dd = 0.0 if variant == "bwd_drop_D" else (p * dp).sum(axis=1)[:, None]
                ds = p * (dp - dd)
                dq[b, h] = (1.0 if variant == "bwd_dq_unscaled" else scale) * (ds @ k[b, hk])
                dk[b, hk] += scale * ((ds @ q[b, h]) if variant == "bwd_dk_not_transposed"
                                      and ds.shape[0] == ds.shape[1] else ds.T @ q[b, h])
                dv[b, hk] += (p @ do[b, h] if variant == "bwd_dv_p_not_transposed"
                              and p.shape[0] == p.shape[1] else p.T @ do[b, h])
                if variant == "bwd_gqa_last_head_only" and rep > 1 and h % rep != rep - 1:
                    dk[b, hk] *= 0.0
                    dv[b, hk] *= 0.0
        return dq, dk, dv
    return attention_backward


MUTATIONS = {
    "scale_squared": ("score_matrix", _scores),
    "drop_bias": ("score_matrix", _scores),
    "bias_scaled": ("score_matrix", _scores),
    "kv_len_off_by_one": ("score_matrix", _scores),
    "causal_top_left": ("score_matrix", _scores),
    "causal_diag_masked": ("score_matrix", _scores),
    "window_top_left": ("score_matrix", _scores),
    "window_sides_swapped": ("score_matrix", _scores),
    "window_left_exclusive": ("score_matrix", _scores),
    "window_drop_right": ("score_matrix", _scores),
    "no_dead_row_guard": ("masked_softmax", _softmax),
    "sign_flip": ("masked_softmax", _softmax),
    "pv_transposed": ("_head_forward", _head),
    "lse_log2": ("_head_forward", _head),
    "lse_drops_max": ("_head_forward", _head),
    "blocked_no_rescale_l": ("online_softmax_blocked", _blocked),
    "blocked_no_rescale_a": ("online_softmax_blocked", _blocked),
    "scalar_no_rescale_a": ("online_softmax_scalar", _scalar),
    "merge_plain_mean": ("merge_partials", _merge),
    "varlen_keys_from_query_offsets": ("attention_varlen", _varlen),
    "bwd_drop_D": ("attention_backward", _backward),
    "bwd_dq_unscaled": ("attention_backward", _backward),
    "bwd_dk_not_transposed": ("attention_backward", _backward),
    "bwd_dv_p_not_transposed": ("attention_backward", _backward),
    "bwd_gqa_last_head_only": ("attention_backward", _backward),
    "varlen_keys_of_all_sequences": ("attention_varlen", _varlen),
}


def _pin_functions():
    return [f for name, f in inspect.getmembers(pins, inspect.isfunction)
            if name.startswith("test_")]


def test_unmutated_oracle_passes_every_pin():
    for f in _pin_functions():
        f()


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_mutation(mutation, monkeypatch):
    fname, maker = MUTATIONS[mutation]
    bad = maker(mutation)
    monkeypatch.setattr(oa, fname, bad)
    if hasattr(oracle, fname):
        monkeypatch.setattr(oracle, fname, bad)
    caught = []
    with np.errstate(all="ignore"):
        for f in _pin_functions():
            try:
                f()
            except Exception as exc:  # AssertionError or a numerical blow-up
                caught.append((f.__name__, type(exc).__name__))
    assert caught, f"no pin notices the planted mistake {mutation!r}"
