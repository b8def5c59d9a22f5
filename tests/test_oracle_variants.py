"""Pins for the serving-side variants of the oracle (CPU only).

The checks use properties the definition fixes, not the oracle's own code
paths: constant value rows (the output of a head is the value its group
reads), equality with the plain multi-head oracle on explicitly repeated K/V
heads, what bottom-right causal alignment implies for a single query, for
N_q > N_k and for the last row, per-sequence decomposition of a packed batch,
and exactness of the split-KV merge (and agreement with the pages' state
form of the combine rule, pinned in test_oracle.py).
"""
import numpy as np
import pytest

from oracle.attention import attention, attention_head, causal_mask, combine
from oracle.variants import attention_gqa, attention_varlen, merge_lse_states, split_states, window_mask


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_gqa_head_mapping_is_floor_division():
    # value rows of KV head kh are all equal to kh + 1, so every output row of
    # query head h equals the index + 1 of the KV head it reads
    B, nq, nk, hq, hkv, d = 1, 5, 7, 6, 3, 4
    q, k = _rand((B, nq, hq, d), 1), _rand((B, nk, hkv, d), 2)
    v = np.zeros((B, nk, hkv, d))
    for kh in range(hkv):
        v[:, :, kh] = kh + 1
    o, _ = attention_gqa(q, k, v, 0.5, False)
    for h in range(hq):
        np.testing.assert_allclose(o[:, :, h], h // (hq // hkv) + 1, rtol=1e-14)


@pytest.mark.parametrize("hkv", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_on_repeated_heads(hkv, causal):
    B, nq, nk, hq, d = 2, 9, 13, 4, 8
    q, k, v = _rand((B, nq, hq, d), 3), _rand((B, nk, hkv, d), 4), _rand((B, nk, hkv, d), 5)
    o, lse = attention_gqa(q, k, v, 0.3, causal)
    # MHA on K/V with every KV head repeated g times along the head axis;
    # plain per-head definition with N_q != N_k
    kr, vr = np.repeat(k, hq // hkv, axis=2), np.repeat(v, hq // hkv, axis=2)
    for b in range(B):
        for h in range(hq):
            oh, lh = attention_head(q[b, :, h], kr[b, :, h], vr[b, :, h], 0.3, causal)
            np.testing.assert_allclose(o[b, :, h], oh, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], lh, rtol=1e-13)
    if nq == nk:
        o2, l2 = attention(q, kr, vr, 0.3, causal)
        np.testing.assert_allclose(o, o2, rtol=1e-13)


def test_single_query_causal_equals_full():
    # bottom-right alignment: with one query the row is the last one and sees
    # every key, so decode under the causal flag is full attention
    q, k, v = _rand((1, 6), 6), _rand((40, 6), 7), _rand((40, 6), 8)
    o1, l1 = attention_head(q, k, v, 0.4, True)
    o2, l2 = attention_head(q, k, v, 0.4, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    # brute force over the keys, pure Python
    s = [0.4 * sum(q[0, t] * k[j, t] for t in range(6)) for j in range(40)]
    mx = max(s)
    w = [np.exp(x - mx) for x in s]
    ref = [sum(w[j] * v[j, t] for j in range(40)) / sum(w) for t in range(6)]
    np.testing.assert_allclose(o1[0], ref, rtol=1e-12)
    np.testing.assert_allclose(l1[0], mx + np.log(sum(w)), rtol=1e-13)


def test_more_queries_than_keys_causal():
    # N_q = 10 > N_k = 4: row i sees keys j <= i - 6; rows 0..5 see nothing,
    # and rows 6..9 are square causal attention of the last 4 queries
    q, k, v = _rand((10, 5), 9), _rand((4, 5), 10), _rand((4, 5), 11)
    o, lse = attention_head(q, k, v, 0.7, True)
    np.testing.assert_array_equal(o[:6], 0.0)
    assert np.all(lse[:6] == -np.inf)
    o2, l2 = attention_head(q[6:], k, v, 0.7, True)
    np.testing.assert_allclose(o[6:], o2, rtol=1e-14)
    np.testing.assert_allclose(lse[6:], l2, rtol=1e-14)
    # the last row sees every key
    o3, _ = attention_head(q[-1:], k, v, 0.7, False)
    np.testing.assert_allclose(o[-1:], o3, rtol=1e-14)


def test_varlen_is_per_sequence_and_handles_empty():
    hq, hkv, d = 4, 2, 8
    lq = [3, 0, 7, 1, 5]
    lk = [5, 4, 7, 0, 2]
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    q = _rand((cu_q[-1], hq, d), 12)
    k, v = _rand((cu_k[-1], hkv, d), 13), _rand((cu_k[-1], hkv, d), 14)
    for causal in (False, True):
        o, lse = attention_varlen(q, k, v, cu_q, cu_k, 0.35, causal)
        assert lse.shape == (hq, cu_q[-1])
        for b in range(len(lq)):
            sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            ob, lb = attention_gqa(q[None, sq], k[None, sk], v[None, sk], 0.35, causal)
            np.testing.assert_allclose(o[sq], ob[0], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(lse[:, sq], lb[0], rtol=1e-13)
        # sequence 3 has a query but no key: O = 0, LSE = -inf
        np.testing.assert_array_equal(o[cu_q[3]:cu_q[4]], 0.0)
        assert np.all(lse[:, cu_q[3]:cu_q[4]] == -np.inf)


def test_varlen_with_equal_lengths_is_the_dense_batch():
    B, n, h, d = 3, 6, 2, 4
    q, k, v = _rand((B, n, h, d), 15), _rand((B, n, h, d), 16), _rand((B, n, h, d), 17)
    cu = np.arange(B + 1) * n
    o, lse = attention_varlen(q.reshape(B * n, h, d), k.reshape(B * n, h, d), v.reshape(B * n, h, d),
                              cu, cu, 0.5, True)
    o2, l2 = attention(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, o2.reshape(B * n, h, d), rtol=1e-14)
    # (H, total) against (B, H, N)
    np.testing.assert_allclose(lse, l2.transpose(1, 0, 2).reshape(h, B * n), rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [1, 5, 12])
def test_split_merge_equals_full(causal, nq):
    nk, d = 23, 6
    q, k, v = _rand((nq, d), 18), _rand((nk, d), 19), _rand((nk, d), 20)
    o_ref, l_ref = attention_head(q, k, v, 0.6, causal)
    for bounds in ([(0, nk)], [(0, 8), (8, 16), (16, 23)], [(0, 1), (1, 20), (20, 23), (23, 23)],
                   [(0, 4)] + [(4 + 4 * i, 8 + 4 * i) for i in range(4)] + [(20, 23)]):
        op, lp = split_states(q, k, v, 0.6, causal, bounds)
        o, lse = merge_lse_states(op, lp)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, l_ref, rtol=1e-12)
        # merge order does not matter
        o2, l2 = merge_lse_states(op[::-1], lp[::-1])
        np.testing.assert_allclose(o2, o_ref, rtol=1e-12, atol=1e-14)
    if causal and nq == 12:
        # keys 20..22 are visible to rows i >= 20 - 11 = 9 only
        op, lp = split_states(q, k, v, 0.6, True, [(20, 23)])
        assert np.all(lp[0, :9] == -np.inf) and np.all(op[0, :9] == 0.0)
        assert np.all(np.isfinite(lp[0, 9:]))


def test_lse_merge_agrees_with_state_combine():
    # the pages' (m, l, O~) rule on the same two key ranges
    nq, nk, d = 7, 16, 5
    q, k, v = _rand((nq, d), 21), _rand((nk, d), 22), _rand((nk, d), 23)
    s = 0.5 * q @ k.T
    states = []
    for k0, k1 in ((0, 9), (9, 16)):
        m = s[:, k0:k1].max(axis=1)
        p = np.exp(s[:, k0:k1] - m[:, None])
        states.append((m, p.sum(axis=1), p @ v[k0:k1]))
    m, l, ot = combine(*states)
    op, lp = split_states(q, k, v, 0.5, False, [(0, 9), (9, 16)])
    o, lse = merge_lse_states(op, lp)
    np.testing.assert_allclose(o, ot / l[:, None], rtol=1e-13)
    np.testing.assert_allclose(lse, m + np.log(l), rtol=1e-13)


def test_window_mask_by_hand():
    # N_q = 3, N_k = 5 (off = 2), window (1, 0): row i sees keys i+1 .. i+2
    m = window_mask(3, 5, 1, 0)
    expect = np.array([[1, 0, 0, 1, 1],
                       [1, 1, 0, 0, 1],
                       [1, 1, 1, 0, 0]], dtype=bool)
    np.testing.assert_array_equal(m, expect)
    # unbounded left, right bound 0: the causal mask
    np.testing.assert_array_equal(window_mask(4, 7, -1, 0), causal_mask(4, 7))
    # both unbounded: nothing excluded
    assert not window_mask(3, 5).any()


def test_window_zero_width_picks_the_diagonal_key():
    # window (0, 0): query i sees only key i + off, so O_i = V_{i+off} and
    # LSE_i = alpha q_i . k_{i+off}
    B, nq, nk, h, d = 1, 4, 9, 2, 5
    q, k, v = _rand((B, nq, h, d), 24), _rand((B, nk, h, d), 25), _rand((B, nk, h, d), 26)
    o, lse = attention_gqa(q, k, v, 0.3, False, window=(0, 0))
    off = nk - nq
    for i in range(nq):
        np.testing.assert_allclose(o[0, i], v[0, i + off], rtol=1e-14)
        for hh in range(h):
            np.testing.assert_allclose(lse[0, hh, i], 0.3 * q[0, i, hh] @ k[0, i + off, hh], rtol=1e-13)


def test_window_brute_force_and_limits():
    nq, nk, d = 6, 10, 3
    q, k, v = _rand((1, nq, 1, d), 27), _rand((1, nk, 1, d), 28), _rand((1, nk, 1, d), 29)
    wl, wr = 2, 1
    o, lse = attention_gqa(q, k, v, 0.5, False, window=(wl, wr))
    off = nk - nq
    for i in range(nq):
        keys = [j for j in range(nk) if i + off - wl <= j <= i + off + wr]
        s = [0.5 * sum(q[0, i, 0, t] * k[0, j, 0, t] for t in range(d)) for j in keys]
        mx = max(s)
        w = [np.exp(x - mx) for x in s]
        ref = [sum(w[a] * v[0, j, 0, t] for a, j in enumerate(keys)) / sum(w) for t in range(d)]
        np.testing.assert_allclose(o[0, i, 0], ref, rtol=1e-12)
    # a window wider than the sequence is full attention; causal with a
    # right window is the causal result
    o1, l1 = attention_gqa(q, k, v, 0.5, False, window=(nk, nk))
    o2, l2 = attention_gqa(q, k, v, 0.5, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    o3, _ = attention_gqa(q, k, v, 0.5, True, window=(-1, 3))
    o4, _ = attention_gqa(q, k, v, 0.5, True)
    np.testing.assert_allclose(o3, o4, rtol=1e-14)
