"""Serving-side variants of the forward, plain float64 (test infrastructure only).

Each variant is the plain definition of ``oracle.attention.attention_head``
applied with different index bookkeeping; nothing here is blocked or fused.

Sources (pages on FlashAttention-3):

* grouped / multi-query attention: "FlashAttention-3 on Hopper", section
  5.6.1: with g query heads per key/value head, query head h reads key/value
  head floor(h / g). (MQA is the case of one key/value head.)
* N_q != N_k: section 4.7 of the same page, causal predicate
  col > row + (N_k - N_q) (bottom-right alignment), as in ``causal_mask``.
* variable-length batches: chapter 9.3 of the same page survives only as a
  heading. Reading taken here: the sequences of a batch are concatenated
  along the token axis; ``cu_seqlens`` holds the B + 1 prefix offsets
  (sequence b owns rows cu[b] .. cu[b+1]-1), and each sequence is an
  independent attention problem with its own N_q, N_k and causal offset.
  LSE is laid out (H_q, total_q).
* local (sliding-window) attention: section 4.7 of the same page says a
  window adds a left boundary to the causal right one; its text gives no
  formula. Reading taken here, with the same bottom-right alignment
  (off = N_k - N_q): query i sees key j iff
  i + off - w_left <= j <= i + off + w_right, a negative width meaning no
  bound on that side; the causal flag is the right bound 0.
* split-KV: section 3.2.1 (the block-combine rule merges the states of
  disjoint key sets) and chapter 10 (split-KV, body missing). Reading taken
  here: the keys are cut into consecutive ranges; the state of one range is
  the plain definition restricted to those keys under the full problem's
  mask, reported normalised, O_s = O~_s / l_s and LSE_s = m_s + ln l_s (an
  empty range gives O_s = 0, LSE_s = -inf). Since l_s = e^(LSE_s - m_s), the
  union of ranges has LSE = ln sum_s e^(LSE_s) and O = sum_s e^(LSE_s - LSE)
  O_s, which is the pages' rule rewritten in these units.

Layouts: dense q (B, N_q, H_q, d), k and v (B, N_k, H_kv, d); O like q; LSE
(B, H_q, N_q). Varlen: q (total_q, H_q, d), k and v (total_k, H_kv, d); O
like q; LSE (H_q, total_q).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head, causal_mask

__all__ = ["window_mask", "attention_gqa", "attention_varlen", "split_states", "merge_lse_states"]


def window_mask(nq, nk, window_left=-1, window_right=-1):
    """(nq, nk) boolean array, True where key j lies outside the window of
    query i: j < i + off - window_left or j > i + off + window_right, with
    off = nk - nq; a negative width leaves that side unbounded."""
    rows = np.arange(nq)[:, None] + (nk - nq)
    cols = np.arange(nk)[None, :]
    out = np.zeros((nq, nk), dtype=bool)
    if window_left >= 0:
        out |= cols < rows - window_left
    if window_right >= 0:
        out |= cols > rows + window_right
    return out


def _group(hq: int, hkv: int) -> int:
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"H_q = {hq} is not a multiple of H_kv = {hkv}")
    return hq // hkv


def attention_gqa(q, k, v, alpha=None, causal=False, window=(-1, -1)):
    """Dense forward with H_q query heads over H_kv key/value heads;
    ``window`` = (w_left, w_right) as in ``window_mask``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, hq, d = q.shape
    hkv = k.shape[2]
    g = _group(hq, hkv)
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    o = np.zeros((B, nq, hq, v.shape[3]))
    lse = np.zeros((B, hq, nq))
    mask = window_mask(nq, k.shape[1], *window)
    for b in range(B):
        for h in range(hq):
            kh = h // g  # section 5.6.1: KV head floor(h / g)
            o[b, :, h], lse[b, h] = attention_head(q[b, :, h], k[b, :, kh], v[b, :, kh], alpha, causal,
                                                   mask=mask)
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, alpha=None, causal=False, window=(-1, -1)):
    """Packed variable-length forward: sequence b is rows cu[b] .. cu[b+1]-1."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    g = _group(hq, hkv)
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    o = np.zeros((tq, hq, v.shape[2]))
    lse = np.full((hq, tq), -np.inf)
    for b in range(cu_q.size - 1):
        q0, q1 = cu_q[b], cu_q[b + 1]
        k0, k1 = cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        mask = window_mask(q1 - q0, k1 - k0, *window)
        for h in range(hq):
            kh = h // g
            o[q0:q1, h], lse[h, q0:q1] = attention_head(q[q0:q1, h], k[k0:k1, kh], v[k0:k1, kh], alpha, causal,
                                                        mask=mask)
    return o, lse


def split_states(q, k, v, alpha, causal, bounds):
    """Normalised states of one head over the key ranges ``bounds``.

    q (N_q, d), k (N_k, d), v (N_k, dv); ``bounds`` is a list of (k0, k1)
    key ranges. Returns (O_parts (S, N_q, dv), LSE_parts (S, N_q)). The mask
    is that of the whole problem (N_q queries against N_k keys).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    s_all = alpha * (q @ k.T)
    if causal:
        s_all = np.where(causal_mask(nq, nk), -np.inf, s_all)
    o_parts = np.zeros((len(bounds), nq, v.shape[1]))
    lse_parts = np.full((len(bounds), nq), -np.inf)
    for i, (k0, k1) in enumerate(bounds):
        if k1 <= k0:
            continue
        s = s_all[:, k0:k1]
        m = s.max(axis=1)
        live = np.isfinite(m)
        m_safe = np.where(live, m, 0.0)
        e = np.exp(s - m_safe[:, None])
        l = e.sum(axis=1)
        ok = live & (l > 0)
        o_parts[i, ok] = (e[ok] / l[ok, None]) @ v[k0:k1]
        lse_parts[i, ok] = m_safe[ok] + np.log(l[ok])
    return o_parts, lse_parts


def merge_lse_states(o_parts, lse_parts):
    """Merge normalised states (O_s, LSE_s) over disjoint key sets.

    o_parts (S, ..., dv), lse_parts (S, ...). LSE = ln sum_s e^(LSE_s),
    O = sum_s e^(LSE_s - LSE) O_s; a row whose every LSE_s is -inf gives
    O = 0 and LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    live = np.isfinite(mx)
    mx_safe = np.where(live, mx, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - mx_safe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(live, mx_safe + np.log(np.where(live, tot, 1.0)), -np.inf)
    frac = np.where(live, w / np.where(live, tot, 1.0), 0.0)
    o = np.einsum("s...,s...d->...d", frac, o_parts)
    return o, lse
