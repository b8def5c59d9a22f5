"""Pins for the float64 attention oracle.

Each check ties the oracle to something other than itself: a library routine
(scipy's softmax / logsumexp), a closed form, an invariance the definition
implies, or brute-force scalar loops. A plausible slip in the oracle (a
dropped alpha, a wrong sign, a transposed operand, a wrong mask direction, a
missing rescale in the recurrence) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special

from oracle.attention import (attention, attention_head, attention_rows, causal_mask, combine,
                              online_attention)
from synth_inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_qkv

TOL = 1e-12


def _rand(n, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)) * scale


def test_probabilities_match_scipy_softmax_and_rows_sum_to_one():
    # With V = I (dv = Nk) the output row is the probability row itself.
    q, k = _rand(7, 5, 1), _rand(9, 5, 2)
    alpha = 0.37
    o, lse = attention_head(q, k, np.eye(9), alpha)
    ref = scipy.special.softmax(alpha * q @ k.T, axis=1)
    np.testing.assert_allclose(o, ref, atol=TOL, rtol=0)
    np.testing.assert_allclose(o.sum(axis=1), 1.0, atol=TOL)
    assert (o >= 0).all()
    np.testing.assert_allclose(lse, scipy.special.logsumexp(alpha * q @ k.T, axis=1), atol=TOL)


def test_causal_probabilities_match_masked_scipy_softmax():
    q, k = _rand(6, 4, 3), _rand(6, 4, 4)
    o, lse = attention_head(q, k, np.eye(6), 0.5, causal=True)
    s = 0.5 * q @ k.T
    s[np.triu_indices(6, 1)] = -np.inf
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1), atol=TOL)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), atol=TOL)
    assert np.all(o[np.triu_indices(6, 1)] == 0)


def test_constant_row_v_gives_the_constant():
    q, k = _rand(11, 8, 5), _rand(13, 8, 6)
    c = np.array([1.5, -2.0, 0.25])
    v = np.tile(c, (13, 1))
    o, _ = attention_head(q, k, v, 0.3)
    np.testing.assert_allclose(o, np.tile(c, (11, 1)), atol=TOL)
    o, _ = attention_head(_rand(13, 8, 7), k, v, 0.3, causal=True)
    np.testing.assert_allclose(o, np.tile(c, (13, 1)), atol=TOL)


def test_joint_key_value_permutation_leaves_output_unchanged():
    q, k, v = _rand(10, 6, 8), _rand(17, 6, 9), _rand(17, 3, 10)
    perm = np.random.default_rng(11).permutation(17)
    o1, l1 = attention_head(q, k, v, 0.4)
    o2, l2 = attention_head(q, k[perm], v[perm], 0.4)
    np.testing.assert_allclose(o1, o2, atol=TOL)
    np.testing.assert_allclose(l1, l2, atol=TOL)
    # permuting keys alone (a transposed or mis-indexed V) must change it
    o3, _ = attention_head(q, k[perm], v, 0.4)
    assert np.abs(o3 - o1).max() > 1e-3


def test_causal_first_row_is_v0_and_lse0_is_the_single_score():
    q, k, v = _rand(8, 5, 12), _rand(8, 5, 13), _rand(8, 5, 14)
    o, lse = attention_head(q, k, v, 0.7, causal=True)
    np.testing.assert_allclose(o[0], v[0], atol=TOL)
    assert abs(lse[0] - 0.7 * q[0] @ k[0]) < TOL


def test_single_key_closed_form():
    q, k, v = _rand(3, 4, 15), _rand(1, 4, 16), _rand(1, 4, 17)
    o, lse = attention_head(q, k, v, 0.9)
    np.testing.assert_allclose(o, np.tile(v[0], (3, 1)), atol=TOL)
    np.testing.assert_allclose(lse, 0.9 * (q @ k[0]), atol=TOL)


def test_zero_queries_give_mean_and_prefix_mean():
    n = 9
    q, k, v = np.zeros((n, 4)), _rand(n, 4, 18), _rand(n, 3, 19)
    o, lse = attention_head(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), atol=TOL)
    np.testing.assert_allclose(lse, math.log(n), atol=TOL)
    o, lse = attention_head(q, k, v, 1.0, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, atol=TOL)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), atol=TOL)


def test_key_shift_moves_lse_by_alpha_q_dot_u_and_keeps_output():
    q, k, v = _rand(6, 5, 20), _rand(12, 5, 21), _rand(12, 5, 22)
    u = _rand(1, 5, 23)[0]
    alpha = 0.6
    o1, l1 = attention_head(q, k, v, alpha)
    o2, l2 = attention_head(q, k + u[None, :], v, alpha)
    np.testing.assert_allclose(o1, o2, atol=1e-11)
    np.testing.assert_allclose(l2 - l1, alpha * q @ u, atol=1e-11)


def test_dominant_score_selects_its_value_row():
    q = np.zeros((1, 4)); q[0, 0] = 1.0
    k = np.zeros((5, 4)); k[3, 0] = 1000.0
    v = _rand(5, 3, 24)
    o, lse = attention_head(q, k, v, 1.0)
    np.testing.assert_allclose(o[0], v[3], atol=1e-12)
    assert abs(lse[0] - 1000.0) < 1e-9


def _brute(q, k, v, alpha, causal):
    nq, nk, dv = len(q), len(k), len(v[0])
    out, lse = [], []
    for i in range(nq):
        s = []
        for j in range(nk):
            if causal and j > i + (nk - nq):
                continue
            s.append((j, alpha * sum(q[i][t] * k[j][t] for t in range(len(q[i])))))
        if not s:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        m = max(x for _, x in s)
        w = [(j, math.exp(x - m)) for j, x in s]
        z = sum(x for _, x in w)
        out.append([sum(x * v[j][c] for j, x in w) / z for c in range(dv)])
        lse.append(m + math.log(z))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("nq,nk,d,causal", [(1, 1, 3, False), (5, 5, 4, True), (8, 8, 2, False),
                                            (3, 7, 5, True), (7, 3, 4, True), (6, 8, 3, False)])
def test_brute_force_scalar_loops(nq, nk, d, causal):
    q, k, v = _rand(nq, d, 30 + nq), _rand(nk, d, 40 + nk), _rand(nk, 3, 50 + nk)
    alpha = 1 / math.sqrt(d)
    o, lse = attention_head(q, k, v, alpha, causal=causal)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), alpha, causal)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)


def test_fully_masked_rows_give_zero_output_and_minus_inf_lse():
    # Bottom-right causal alignment with more queries than keys: the first
    # nq - nk rows see no key at all.
    q, k, v = _rand(7, 4, 60), _rand(3, 4, 61), _rand(3, 4, 62)
    o, lse = attention_head(q, k, v, 0.5, causal=True)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[:4]))
    assert np.all(np.isfinite(lse[4:]))
    np.testing.assert_allclose(o[4], v[0], atol=TOL)  # row 4 sees only key 0


def test_causal_mask_is_bottom_right_aligned():
    m = causal_mask(2, 4)
    assert m.tolist() == [[False, False, False, True], [False, False, False, False]]
    assert causal_mask(3, 3).tolist() == [[False, True, True], [False, False, True], [False, False, False]]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_online_recurrence_equals_definition_in_any_tile_order(block, causal):
    n, d = 37, 8
    q, k, v = _rand(n, d, 70), _rand(n, d, 71), _rand(n, d, 72)
    o, lse = attention_head(q, k, v, 0.35, causal=causal)
    nb = (n + block - 1) // block
    for order in (range(nb), range(nb - 1, -1, -1), np.random.default_rng(block).permutation(nb)):
        o2, l2 = online_attention(q, k, v, 0.35, causal=causal, block=block, order=order)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(l2, lse, atol=1e-12)


def test_block_combine_of_disjoint_halves_equals_full():
    q, k, v = _rand(5, 6, 80), _rand(20, 6, 81), _rand(20, 4, 82)
    alpha = 0.45

    def state(ks, vs):
        s = alpha * q @ ks.T
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        return m, p.sum(axis=1), p @ vs

    m, l, ot = combine(state(k[:7], v[:7]), state(k[7:], v[7:]))
    o, lse = attention_head(q, k, v, alpha)
    np.testing.assert_allclose(ot / l[:, None], o, atol=TOL)
    np.testing.assert_allclose(m + np.log(l), lse, atol=TOL)
    # a side with no visible key contributes nothing
    empty = (np.full(5, -np.inf), np.zeros(5), np.zeros((5, 4)))
    m2, l2, o2 = combine(state(k, v), empty)
    np.testing.assert_allclose(o2 / l2[:, None], o, atol=TOL)


def test_full_tensor_layout_and_default_alpha():
    bits, (q, k, v) = make_qkv(2, 19, 3, 8, seed=5)
    o, lse = attention(q, k, v, causal=True)
    assert o.shape == (2, 19, 3, 8) and lse.shape == (2, 3, 19)
    ob, lb = attention_head(q[1, :, 2], k[1, :, 2], v[1, :, 2], 1 / math.sqrt(8), causal=True)
    np.testing.assert_allclose(o[1, :, 2], ob, atol=TOL)
    np.testing.assert_allclose(lse[1, 2], lb, atol=TOL)
    rows = np.array([0, 5, 18])
    (os_, ls_), = attention_rows(q, k, v, 1 / math.sqrt(8), True, [(1, 2, rows)])
    np.testing.assert_allclose(os_, ob[rows], atol=TOL)
    np.testing.assert_allclose(ls_, lb[rows], atol=TOL)


def test_row_chunking_does_not_change_results():
    q, k, v = _rand(50, 4, 90), _rand(50, 4, 91), _rand(50, 4, 92)
    a = attention_head(q, k, v, 0.5, causal=True, row_chunk=7)
    b = attention_head(q, k, v, 0.5, causal=True, row_chunk=1024)
    # BLAS may block the products differently per chunk shape: rounding only
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_bf16_rounding_matches_torch_cpu():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    mine = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeded_inputs_are_reproducible_and_standard_normal():
    b1, v1 = make_qkv(1, 64, 2, 64, seed=0)
    b2, v2 = make_qkv(1, 64, 2, 64, seed=0)
    for x, y in zip(b1, b2):
        np.testing.assert_array_equal(x, y)
    allv = np.concatenate([t.ravel() for t in v1])
    assert abs(allv.mean()) < 0.05 and abs(allv.std() - 1) < 0.05
    b3, _ = make_qkv(1, 64, 2, 64, seed=1)
    assert not np.array_equal(b1[0], b3[0])


def test_golden_tiny_fixture():
    """Regression record of the oracle (tests/golden/make_golden.py), with the
    hand-checkable entries re-derived here: causal row 0 is V[0] with
    LSE = alpha * q0.k0; every full row's LSE is ln sum_j exp(alpha q.k_j)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_attention.json")
    g = json.load(open(path))
    q, k, v = (np.array(g[n], float) for n in ("Q", "K", "V"))
    a = g["alpha"]
    assert g["causal"]["O"][0] == g["V"][0]
    assert abs(g["causal"]["LSE"][0] - a * q[0] @ k[0]) < 1e-15
    for i in range(3):
        assert abs(g["full"]["LSE"][i] - math.log(sum(math.exp(a * q[i] @ k[j]) for j in range(3)))) < 1e-14
    for causal, key in ((False, "full"), (True, "causal")):
        o, lse = attention_head(q, k, v, a, causal=causal)
        np.testing.assert_allclose(o, g[key]["O"], atol=1e-14)
        np.testing.assert_allclose(lse, g[key]["LSE"], atol=1e-14)
