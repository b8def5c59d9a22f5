"""Pins for the backward oracle (CPU only).

Each check is independent of the formulas the oracle is written with (section
7.1 of "FlashAttention-3 on Hopper"): central finite differences of the
forward oracle, torch float64 autograd through a plain torch forward (its own
softmax derivative), and invariants of the attention function itself.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attention
from oracle.attention_bwd import attention_backward


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, alpha, causal):
    o, _ = attention(q, k, v, alpha, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    B, N, H, d = 1, 5, 2, 3
    q, k, v, do = (_rand((B, N, H, d), s) for s in range(4))
    alpha = 0.7
    dq, dk, dv = attention_backward(q, k, v, do, alpha, causal)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, alpha, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, alpha, causal)
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    B, N, H, d = 2, 37, 2, 16
    q, k, v, do = (_rand((B, N, H, d), 10 + s) for s in range(4))
    alpha = 1.0 / np.sqrt(d)
    dq, dk, dv = attention_backward(q, k, v, do, alpha, causal)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    # plain torch forward in (B, H, N, d) with torch's own softmax
    qh, kh, vh = (t.permute(0, 2, 1, 3) for t in (tq, tk, tv))
    s = alpha * torch.matmul(qh, kh.transpose(-1, -2).contiguous())
    if causal:
        mask = torch.triu(torch.ones(N, N, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vh).permute(0, 2, 1, 3)
    (o * torch.tensor(do)).sum().backward()
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    B, N, H, d = 2, 19, 3, 8
    q, k, v, do = (_rand((B, N, H, d), 20 + s) for s in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.4, causal)
    # K -> K + 1 u^T shifts every score of row i by alpha q_i.u: O is unchanged,
    # so the gradient along that direction, sum_j dK_j, vanishes
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # rows of P sum to one: sum_j dV_j = sum_j sum_i P_ij dO_i = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


def test_backward_constant_v_and_single_key():
    B, N, H, d = 1, 11, 2, 4
    q, k, do = (_rand((B, N, H, d), 30 + s) for s in range(3))
    v = np.broadcast_to(_rand((B, 1, H, d), 33), (B, N, H, d)).copy()
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, False)
    # every output row equals the constant row: O does not depend on Q or K
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    # one key: O = V_0, so dV_0 = dO_0 and dQ = dK = 0
    q1, k1, v1, do1 = (x[:, :1] for x in (q, k, _rand((B, N, H, d), 34), do))
    dq1, dk1, dv1 = attention_backward(q1, k1, v1, do1, 0.5, False)
    np.testing.assert_allclose(dv1, do1, atol=1e-15)
    np.testing.assert_allclose(dq1, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk1, 0.0, atol=1e-15)


def test_backward_causal_first_row_and_row_chunks():
    B, N, H, d = 1, 29, 1, 8
    q, k, v, do = (_rand((B, N, H, d), 40 + s) for s in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, 0.3, True)
    # causal row 0 sees only key 0 (O_0 = V_0): its query gets no gradient
    np.testing.assert_allclose(dq[:, 0], 0.0, atol=1e-15)
    # the last key is seen only by the last row
    s = 0.3 * q[0, -1, 0] @ k[0, :, 0].T
    p_last = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
    np.testing.assert_allclose(dv[0, -1, 0], p_last[-1] * do[0, -1, 0], rtol=1e-12)
    # chunking the rows does not change the result
    g1 = attention_backward(q, k, v, do, 0.3, True, row_chunk=7)
    for a, b in zip((dq, dk, dv), g1):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(3, 6), (6, 3)])
def test_gqa_backward_matches_central_differences(causal, nq, nk):
    # 4 query heads over 2 KV heads, N_q != N_k (bottom-right causal): the
    # gradients of sum(O o dO), O from the GQA forward oracle, by differences
    from oracle.attention_bwd import attention_backward_gqa
    from oracle.variants import attention_gqa
    B, hq, hkv, d = 1, 4, 2, 3
    q, do = _rand((B, nq, hq, d), 50), _rand((B, nq, hq, d), 51)
    k, v = _rand((B, nk, hkv, d), 52), _rand((B, nk, hkv, d), 53)
    alpha = 0.6
    dq, dk, dv = attention_backward_gqa(q, k, v, do, alpha, causal)

    def loss(q_, k_, v_):
        o, _ = attention_gqa(q_, k_, v_, alpha, causal)
        return float(np.sum(o * do))
    eps = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_gqa_backward_with_one_group_is_mha():
    from oracle.attention_bwd import attention_backward_gqa
    B, N, H, d = 2, 9, 3, 4
    q, k, v, do = (_rand((B, N, H, d), 60 + s) for s in range(4))
    for causal in (False, True):
        a = attention_backward_gqa(q, k, v, do, 0.5, causal)
        b = attention_backward(q, k, v, do, 0.5, causal)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("window", [(1, 0), (2, 1), (-1, 1), (0, -1)])
def test_windowed_backward_matches_central_differences(window):
    from oracle.attention_bwd import attention_backward_gqa
    from oracle.variants import attention_gqa
    B, nq, nk, hq, hkv, d = 1, 5, 7, 2, 1, 3
    q, do = _rand((B, nq, hq, d), 70), _rand((B, nq, hq, d), 71)
    k, v = _rand((B, nk, hkv, d), 72), _rand((B, nk, hkv, d), 73)
    dq, dk, dv = attention_backward_gqa(q, k, v, do, 0.8, False, window)

    def loss(q_, k_, v_):
        o, _ = attention_gqa(q_, k_, v_, 0.8, False, window=window)
        return float(np.sum(o * do))
    eps = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            fd[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-8, err_msg=f"{name} {window}")


def test_varlen_backward_is_per_sequence():
    from oracle.attention_bwd import attention_backward_gqa, attention_backward_varlen
    lq, lk = [3, 0, 5, 2], [4, 3, 5, 0]
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    hq, hkv, d = 4, 2, 3
    q, do = _rand((cu_q[-1], hq, d), 80), _rand((cu_q[-1], hq, d), 81)
    k, v = _rand((cu_k[-1], hkv, d), 82), _rand((cu_k[-1], hkv, d), 83)
    dq, dk, dv = attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.7, True, (2, 0))
    for b in range(4):
        sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        if lq[b] and lk[b]:
            g = attention_backward_gqa(q[None, sq], k[None, sk], v[None, sk], do[None, sq], 0.7, True, (2, 0))
            np.testing.assert_allclose(dq[sq], g[0][0], rtol=1e-14)
            np.testing.assert_allclose(dk[sk], g[1][0], rtol=1e-14)
        else:
            # a sequence without keys (or queries) has no gradient
            assert np.all(dq[sq] == 0) and np.all(dk[sk] == 0) and np.all(dv[sk] == 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(41, 41), (23, 57), (57, 23)])
def test_sampled_backward_matches_autograd_and_full(causal, nq, nk):
    # row-by-row dQ and column-by-column dK, dV equal torch float64 autograd
    # through a plain softmax, and the full oracle, on every row and key
    from oracle.attention_bwd import attention_backward_head, attention_backward_sampled
    d = 16
    q, do = _rand((nq, d), 21), _rand((nq, d), 22)
    k, v = _rand((nk, d), 23), _rand((nk, d), 24)
    alpha = 0.3
    rows, keys = list(range(nq)), list(range(nk))
    gq, gk, gv = attention_backward_sampled(q, k, v, do, alpha, causal, rows, keys, row_chunk=16)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = alpha * torch.matmul(tq, tk.T.contiguous())
    if causal:
        mask = torch.arange(nk)[None, :] > torch.arange(nq)[:, None] + (nk - nq)
        s = s.masked_fill(mask, float("-inf"))
    pr = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)   # rows with no key: P = 0
    (torch.matmul(pr, tv) * torch.tensor(do)).sum().backward()
    for g, t in ((gq, tq), (gk, tk), (gv, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)
    full = attention_backward_head(q, k, v, do, alpha, causal)
    for g, f in zip((gq, gk, gv), full):
        np.testing.assert_allclose(g, f, rtol=1e-10, atol=1e-12)
