"""Attention forward, plain float64 definition (test infrastructure only).

Sources (pages on FlashAttention-3 and its lineage):

* "FlashAttention-3 paper review" (diycv.top), section on the problem
  background: single-head attention is S = alpha Q K^T, P = softmax(S) taken
  row-wise, O = P V, with alpha typically 1/sqrt(d).
* "FlashAttention-3 on Hopper", section 3.1: masks are represented by
  setting excluded scores to -inf before the softmax; section 4.7: the causal
  predicate masks col > row + (N_k - N_q) (bottom-right alignment);
  section 4.6, finalize step: rows whose normaliser is 0 produce O = 0 and
  LSE = -inf; section 3.4.1 / 4.2: LSE = m + log(l) in natural-log units.
* "FlashAttention-3 on Hopper", section 3.2 and 4.2, and "FlashAttention
  v1-v4" (tom-jerr.github.io), section "先建立共同的计算图": the online state
  (m, l, O~) recurrence, exact in real arithmetic and independent of the tile
  order; section 3.2.1: two states over disjoint key sets combine with the
  same rescaling rule.

The plain definition (``attention``) materialises S and P for one (b, h) and
a chunk of query rows at a time. It is the oracle. ``online_attention`` and
``combine`` restate the pages' streaming algorithm step by step; they exist so
the tests can show that the algorithm reaches the definition, and are never
compared against the GPU in place of it.

Layouts: q, k, v are (B, N, H, d) arrays (d fastest, as the GPU stores them);
O is returned as (B, N, H, d) float64, LSE as (B, H, N) float64.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "attention",
    "attention_head",
    "attention_rows",
    "online_attention",
    "combine",
    "causal_mask",
]


def causal_mask(nq: int, nk: int) -> np.ndarray:
    """Boolean (nq, nk) array, True where a score is excluded.

    "FlashAttention-3 on Hopper", section 4.7: an entry is masked when its
    column exceeds its row plus (N_k - N_q) (bottom-right alignment). With
    N_q = N_k this is the usual "key index > query index".
    """
    rows = np.arange(nq)[:, None]
    cols = np.arange(nk)[None, :]
    return cols > rows + (nk - nq)


def attention_head(q, k, v, alpha, causal=False, row_chunk=1024, rows=None, mask=None):
    """One (batch, head): q (Nq, d), k (Nk, d), v (Nk, dv) -> (O, LSE).

    Follows the plain definition row by row ("FlashAttention-3 paper review",
    problem background; "FlashAttention-3 on Hopper", section 3.1):

    1. S = alpha * q k^T in float64;
    2. masked entries (causal) set to -inf;
    3. m_i = max_j S_ij;
    4. P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i);
    5. O = P v;
    6. LSE_i = m_i + ln sum_j exp(S_ij - m_i);
    7. a row with every entry excluded gives O_i = 0 and LSE_i = -inf
       (section 4.6, finalize).

    ``rows`` optionally selects query rows (an index array); the result then
    has one row per selected index. Rows are processed ``row_chunk`` at a time
    so S never needs more than row_chunk * Nk doubles. ``mask``, when given,
    is a further (Nq, Nk) boolean array of excluded entries (step 2).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.full(rows.size, -np.inf, dtype=np.float64)
    if nk == 0:
        return out, lse
    for start in range(0, rows.size, row_chunk):
        sel = rows[start:start + row_chunk]
        s = float(alpha) * (q[sel] @ k.T)
        if causal:
            s = np.where(causal_mask(nq, nk)[sel], -np.inf, s)
        if mask is not None:
            s = np.where(np.asarray(mask, dtype=bool)[sel], -np.inf, s)
        m = s.max(axis=1)
        live = np.isfinite(m)
        m_safe = np.where(live, m, 0.0)
        e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked entries
        l = e.sum(axis=1)
        ok = live & (l > 0)
        o = np.zeros((sel.size, v.shape[1]))
        o[ok] = (e[ok] / l[ok, None]) @ v
        out[start:start + sel.size] = o
        lse[start:start + sel.size] = np.where(ok, m_safe + np.log(np.where(ok, l, 1.0)), -np.inf)
    return out, lse


def attention(q, k, v, alpha=None, causal=False, row_chunk=1024):
    """Full (B, N, H, d) attention forward in float64: returns (O, LSE).

    O has the layout of q (B, N, H, dv); LSE is (B, H, N). ``alpha`` defaults
    to 1/sqrt(d) (the pages' typical choice; the library takes it as an
    explicit argument).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, H, d = q.shape
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    o = np.zeros((B, nq, H, v.shape[3]), dtype=np.float64)
    lse = np.zeros((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            ob, lb = attention_head(q[b, :, h], k[b, :, h], v[b, :, h], alpha, causal, row_chunk)
            o[b, :, h] = ob
            lse[b, h] = lb
    return o, lse


def attention_rows(q, k, v, alpha, causal, samples):
    """Sampled outputs for large problems.

    ``samples`` is a list of (b, h, rows) triples; returns a list of
    (O_rows, LSE_rows) pairs computed with the plain definition restricted to
    those query rows (the keys are never subsampled).
    """
    res = []
    for b, h, rows in samples:
        res.append(attention_head(q[b, :, h], k[b, :, h], v[b, :, h], alpha, causal, rows=rows))
    return res


def _tile_state(s_tile, v_tile):
    """State (m, l, O~) of one key block on its own (scores already scaled/masked)."""
    m = s_tile.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s_tile - m_safe[:, None])
    return m, p.sum(axis=1), p @ v_tile


def combine(state_a, state_b):
    """Merge two online-softmax states over disjoint key sets.

    "FlashAttention-3 on Hopper", section 3.2.1: with m = max(m_a, m_b), the
    union has l = e^{m_a - m} l_a + e^{m_b - m} l_b and
    O~ = e^{m_a - m} O~_a + e^{m_b - m} O~_b. A side whose maximum is -inf
    (no visible key) contributes nothing.
    """
    ma, la, oa = state_a
    mb, lb, ob = state_b
    m = np.maximum(ma, mb)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    fa = np.where(np.isfinite(ma), np.exp(ma - m_safe), 0.0)
    fb = np.where(np.isfinite(mb), np.exp(mb - m_safe), 0.0)
    return m, fa * la + fb * lb, fa[:, None] * oa + fb[:, None] * ob


def online_attention(q, k, v, alpha, causal=False, block=64, order=None):
    """One head through the streaming (m, l, O~) recurrence.

    "FlashAttention-3 on Hopper", section 4.2 (and "FlashAttention v1-v4",
    "先建立共同的计算图"): start from m = -inf, l = 0, O~ = 0; for each key
    block t (in the given processing order)

        m_t  = max(m_{t-1}, rowmax(S_t))
        rho  = exp(m_{t-1} - m_t)
        P~_t = exp(S_t - m_t)
        l_t  = rho * l_{t-1} + rowsum(P~_t)
        O~_t = rho * O~_{t-1} + P~_t V_t

    and finish with O = O~ / l, LSE = m + log l (section 3.4.1). A row
    whose maximum is still -inf uses 0 as its reference (section 4.6, step 2),
    and a row with l = 0 at the end gives O = 0, LSE = -inf.

    ``order`` is a permutation of the block indices (default: ascending).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    nblocks = (nk + block - 1) // block
    if order is None:
        order = range(nblocks)
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    o = np.zeros((nq, v.shape[1]))
    mask = causal_mask(nq, nk) if causal else None
    for t in order:
        lo, hi = t * block, min(nk, (t + 1) * block)
        s = float(alpha) * (q @ k[lo:hi].T)
        if causal:
            s = np.where(mask[:, lo:hi], -np.inf, s)
        m_new = np.maximum(m, s.max(axis=1))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        rho = np.exp(m - ref)  # exp(-inf) = 0 when nothing was seen yet
        p = np.exp(s - ref[:, None])
        l = rho * l + p.sum(axis=1)
        o = rho[:, None] * o + p @ v[lo:hi]
        m = m_new
    ok = l > 0
    out = np.zeros_like(o)
    out[ok] = o[ok] / l[ok, None]
    lse = np.where(ok, np.where(np.isfinite(m), m, 0.0) + np.log(np.where(ok, l, 1.0)), -np.inf)
    return out, lse
