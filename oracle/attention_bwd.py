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

__all__ = ["attention_backward", "attention_backward_head", "attention_backward_gqa", "attention_backward_varlen"]


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
