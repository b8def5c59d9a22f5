"""Attention backward, plain float64 definition (test infrastructure only).

Sources: "FlashAttention-3 on Hopper", chapter 7 ("The FA3 Backward Pass:
Algorithm"):

* section 7.1: with S = alpha Q K^T, P = softmax(S) row-wise and O = P V, an
  upstream gradient dO gives dV = P^T dO, dP = dO V^T, dS = P o (dP - D) with
  D_i = <P_i, dP_i> (the contracted softmax Jacobian, section 7.1.1),
  dQ = alpha dS K and dK = alpha dS^T Q (product rule on the two GEMMs);
* section 7.1.2: D_i = rowsum(dO_i o O_i), equal to <P_i, dP_i> because
  dP = dO V^T and O = P V;
* masked scores are -inf in S, so their P and dS are 0 and they contribute to
  no gradient (section 3.1 of the same page for the mask convention).

The functions materialise S and P for one (b, h) and a chunk of query rows at
a time. Layouts as in ``oracle.attention``: q, k, v, do are (B, N, H, d);
the gradients are returned as (B, N, H, d) float64.

The GPU backward shares no code with this module.
"""
from __future__ import annotations

import numpy as np

from .attention import causal_mask

__all__ = ["attention_backward", "attention_backward_head", "attention_backward_gqa", "attention_backward_varlen",
           "attention_backward_sampled"]


def attention_backward_head(q, k, v, do, alpha, causal=False, row_chunk=1024, mask=None):
    """Gradients (dq, dk, dv) of one head: q, do are (N_q, d), k, v are
    (N_k, d) float64; causal uses the bottom-right alignment of the forward,
    and ``mask`` is a further (N_q, N_k) boolean array of excluded entries."""
    n = q.shape[0]
    nk = k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = alpha * (q[r0:r1] @ k.T)
        if causal:
            s = np.where(causal_mask(n, nk)[r0:r1], -np.inf, s)
        if mask is not None:
            s = np.where(np.asarray(mask, dtype=bool)[r0:r1], -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        live = np.isfinite(m)
        e = np.where(live, np.exp(s - np.where(live, m, 0.0)), 0.0)
        den = e.sum(axis=1, keepdims=True)
        p = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)
        o = p @ v
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        d_i = np.sum(do[r0:r1] * o, axis=1, keepdims=True)
        ds = p * (dp - d_i)
        dq[r0:r1] = alpha * (ds @ k)
        dk += alpha * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_backward(q, k, v, do, alpha=None, causal=False, row_chunk=1024):
    """Gradients of sum(O o dO) with respect to q, k, v (all (B, N, H, d))."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, N, H, d = q.shape
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            gq, gk, gv = attention_backward_head(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :],
                                                 alpha, causal, row_chunk)
            dq[b, :, h, :] = gq
            dk[b, :, h, :] = gk
            dv[b, :, h, :] = gv
    return dq, dk, dv


def attention_backward_gqa(q, k, v, do, alpha=None, causal=False, window=(-1, -1)):
    """Gradients for H_q query heads over H_kv key/value heads.

    q, do are (B, N_q, H_q, d); k, v are (B, N_k, H_kv, d). Query head h
    reads key/value head floor(h / g) ("FlashAttention-3 on Hopper",
    section 5.6.1), so by the chain rule the gradient of a key/value head is
    the sum of the per-head gradients of the g query heads that read it
    (section 8.8 describes that accumulation).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, nq, hq, d = q.shape
    hkv = k.shape[2]
    if hkv < 1 or hq % hkv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    g = hq // hkv
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    from .variants import window_mask
    mask = window_mask(nq, k.shape[1], *window)
    for b in range(B):
        for h in range(hq):
            kh = h // g
            gq, gk, gv = attention_backward_head(q[b, :, h], k[b, :, kh], v[b, :, kh], do[b, :, h], alpha, causal,
                                                 mask=mask)
            dq[b, :, h] = gq
            dk[b, :, kh] += gk
            dv[b, :, kh] += gv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, alpha=None, causal=False, window=(-1, -1)):
    """Gradients of a packed variable-length batch: q, do (total_q, H_q, d),
    k, v (total_k, H_kv, d); sequence b owns rows cu[b] .. cu[b+1]-1 and is an
    independent problem (the forward's reading of packed batches)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if alpha is None:
        alpha = 1.0 / np.sqrt(q.shape[2])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(cu_q.size - 1):
        sq = slice(cu_q[b], cu_q[b + 1])
        sk = slice(cu_k[b], cu_k[b + 1])
        if cu_q[b + 1] == cu_q[b] or cu_k[b + 1] == cu_k[b]:
            continue
        gq, gk, gv = attention_backward_gqa(q[None, sq], k[None, sk], v[None, sk], do[None, sq], alpha, causal,
                                            window)
        dq[sq], dk[sk], dv[sk] = gq[0], gk[0], gv[0]
    return dq, dk, dv


def attention_backward_sampled(q, k, v, do, alpha, causal=False, rows=(), keys=(), row_chunk=1024):
    """dQ at the query ``rows`` and dK, dV at the ``keys`` of one head, for
    sequences too long to materialise the gradients whole.

    q, do are (N_q, d) and k, v (N_k, d). The same formulas as
    ``attention_backward_head`` (section 7.1 of "FlashAttention-3 on
    Hopper"), taken one output row at a time:

    * a first pass over row chunks gives every row's LSE and
      D_i = rowsum(dO_i o O_i) (section 7.1.2), with O = P V;
    * dQ_i = alpha sum_j P_ij (dP_ij - D_i) K_j for a sampled query i, where
      P_ij = exp(S_ij - LSE_i) and dP_ij = <dO_i, V_j> (P recomputed from the
      LSE, section 7.1.3);
    * dV_j = sum_i P_ij dO_i and dK_j = alpha sum_i P_ij (dP_ij - D_i) Q_i for
      a sampled key j, from column j of P and dP.

    Causal uses the bottom-right alignment; rows with no visible key have
    LSE = -inf and P = 0. Returns (dq_rows, dk_keys, dv_keys) as float64
    arrays of shape (len(rows), d) and (len(keys), d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    off = nk - nq
    lse = np.full(nq, -np.inf)
    dvec = np.zeros(nq)
    for r0 in range(0, nq, row_chunk):
        r1 = min(nq, r0 + row_chunk)
        s = alpha * (q[r0:r1] @ k.T)
        if causal:
            s = np.where(np.arange(nk)[None, :] > np.arange(r0, r1)[:, None] + off, -np.inf, s)
        m = s.max(axis=1, keepdims=True) if nk else np.full((r1 - r0, 1), -np.inf)
        live = np.isfinite(m)
        e = np.where(live, np.exp(s - np.where(live, m, 0.0)), 0.0)
        den = e.sum(axis=1, keepdims=True)
        o = (e / np.where(den > 0, den, 1.0)) @ v
        lse[r0:r1] = np.where(live[:, 0], m[:, 0] + np.log(np.where(den[:, 0] > 0, den[:, 0], 1.0)), -np.inf)
        dvec[r0:r1] = np.sum(do[r0:r1] * o, axis=1)

    def p_of(svals, lrow):
        ok = np.isfinite(svals) & np.isfinite(lrow)
        return np.where(ok, np.exp(np.where(ok, svals - np.where(np.isfinite(lrow), lrow, 0.0), 0.0)), 0.0)

    dq_rows = np.zeros((len(rows), q.shape[1]))
    for n, i in enumerate(rows):
        s = alpha * (k @ q[i])
        if causal:
            s = np.where(np.arange(nk) > i + off, -np.inf, s)
        p = p_of(s, lse[i])
        ds = p * (v @ do[i] - dvec[i])
        dq_rows[n] = alpha * (ds @ k)
    dk_keys = np.zeros((len(keys), k.shape[1]))
    dv_keys = np.zeros((len(keys), v.shape[1]))
    for n, j in enumerate(keys):
        s = alpha * (q @ k[j])
        if causal:
            s = np.where(j > np.arange(nq) + off, -np.inf, s)
        p = p_of(s, lse)
        ds = p * (do @ v[j] - dvec)
        dv_keys[n] = p @ do
        dk_keys[n] = alpha * (ds @ q)
    return dq_rows, dk_keys, dv_keys
