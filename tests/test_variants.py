"""GPU parity of attn_fwd_ex (grouped heads, N_q != N_k, packed batches,
split-KV) against the float64 oracle in ``oracle.variants``.

Inputs come from ``synth_inputs.make_qkv_gqa`` / ``make_seqlens`` (N(0,1)
rounded to bf16 or f16); the oracle consumes the same rounded values.
Tolerances are those of the 16-bit forward (max |dO| <= 1e-2, RMSE <= 3e-3,
|dLSE| <= 1e-3): each key range of a split is the same float32 computation
as the unsplit kernel over fewer keys, and the merge adds float32 rounding
of e^(LSE_s - LSE) (relative 2^-23 per term), far below those bounds. Rows
that see no key must give exactly O = 0 and LSE = -inf.
"""
import numpy as np
import pytest

from gpu_util import assert_bf16_tolerances, errors, to_f64
from oracle.variants import attention_gqa, attention_varlen, split_states
from synth_inputs import make_qkv_gqa, make_seqlens

pytestmark = pytest.mark.gpu


def _dev(bits, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(tdt).cuda() for b in bits]


def _split_len(nk, s):
    # key range length rule of attn_fwd_ex (include/attn.h)
    per = -(-nk // s)
    return -(-per // 64) * 64


def _dense(ea, B, Nq, Nk, Hq, Hkv, d, causal, pack, splits, seed=0, dtype="bf16", alpha=None, window=(-1, -1)):
    import torch
    bits, vals = make_qkv_gqa(B, Nq, Nk, Hq, Hkv, d, seed=seed, dtype=dtype)
    q, k, v = _dev(bits, dtype)
    o, lse = ea.attention_ex(q, k, v, causal=causal, alpha=alpha, pack_gqa=pack, num_splits=splits, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_gqa(*vals, alpha, causal, window=window)
    return to_f64(o), to_f64(lse), o_ref, l_ref


def _check(o, lse, o_ref, l_ref, tag):
    assert np.all(np.isfinite(o)), tag
    # rows with no visible key: exactly zero and -inf
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), dead), tag
    assert_bf16_tolerances(errors(o, o_ref, lse, l_ref), tag)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 1), (3, 3)])
@pytest.mark.parametrize("pack", [0, 1])
def test_gqa_dense(gpu, d, hq, hkv, pack):
    for causal in (False, True):
        o, lse, o_ref, l_ref = _dense(gpu, 2, 150, 150, hq, hkv, d, causal, pack, 1, seed=d + hq)
        _check(o, lse, o_ref, l_ref, (d, hq, hkv, pack, causal))


@pytest.mark.parametrize("nq,nk", [(1, 300), (77, 200), (300, 77), (129, 1), (5, 64), (64, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_nq_ne_nk(gpu, nq, nk, causal):
    o, lse, o_ref, l_ref = _dense(gpu, 2, nq, nk, 4, 2, 128, causal, -1, 1, seed=nq * 7 + nk)
    _check(o, lse, o_ref, l_ref, (nq, nk, causal))
    if causal and nq > nk:
        # the first nq - nk rows of every head see no key
        assert np.all(o[:, : nq - nk] == 0.0)
        assert np.all(np.isneginf(lse[:, :, : nq - nk]))


@pytest.mark.parametrize("nk", [1, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("splits", [1, 3, 8])
def test_decode_split_kv(gpu, nk, splits):
    # one query per sequence (decode), 8 query heads per KV head
    o, lse, o_ref, l_ref = _dense(gpu, 3, 1, nk, 16, 2, 128, True, -1, splits, seed=nk + splits)
    _check(o, lse, o_ref, l_ref, (nk, splits))


@pytest.mark.parametrize("d", [64, 256])
def test_split_kv_other_head_dims_and_f16(gpu, d):
    o, lse, o_ref, l_ref = _dense(gpu, 2, 40, 700, 4, 4, d, True, 0, 5, seed=d, dtype="f16", alpha=0.2)
    _check(o, lse, o_ref, l_ref, d)


def test_split_workspace_holds_the_range_states(gpu):
    import torch
    B, Nq, Nk, Hq, Hkv, d, S = 2, 3, 500, 4, 2, 128, 4
    bits, vals = make_qkv_gqa(B, Nq, Nk, Hq, Hkv, d, seed=3)
    q, k, v = _dev(bits, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
    ws = torch.full((gpu.attn_splitkv_workspace_bytes(S, B * Nq, Hq, d) // 4,), float("nan"), device="cuda")
    gpu.attn_fwd_ex(q, k, v, o, lse, causal=True, pack_gqa=1, num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    sl = _split_len(Nk, S)
    used = -(-Nk // sl)
    bounds = [(s * sl, min(Nk, (s + 1) * sl)) for s in range(used)]
    opart = to_f64(ws[: used * B * Nq * Hq * d]).reshape(used, B, Nq, Hq, d)
    # the LSE block follows the O block of the ranges actually used
    lpart = to_f64(ws[used * B * Nq * Hq * d: used * B * Nq * Hq * (d + 1)]).reshape(used, B, Nq, Hq)
    qv, kv, vv = vals
    alpha = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            op, lp = split_states(qv[b, :, h], kv[b, :, h // (Hq // Hkv)], vv[b, :, h // (Hq // Hkv)], alpha,
                                  True, bounds)
            assert np.abs(opart[:, b, :, h] - op).max() <= 1e-2
            assert np.abs(lpart[:, b, :, h] - lp).max() <= 1e-3


def test_ex_matches_attn_fwd_bitwise(gpu):
    # with Hkv = Hq, Nq = Nk, one range and no packing it is the same kernel
    import torch
    bits, _ = make_qkv_gqa(2, 333, 333, 3, 3, 128, seed=4)
    q, k, v = _dev(bits, "bf16")
    for causal in (False, True):
        o1, l1 = gpu.attention(q, k, v, causal=causal)
        o2, l2 = gpu.attention_ex(q, k, v, causal=causal, pack_gqa=0, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _varlen(ea, lens_q, lens_k, Hq, Hkv, d, causal, splits, pack=-1, seed=0, window=(-1, -1)):
    import torch
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    bits, vals = make_qkv_gqa(1, int(cu_q[-1]), int(cu_k[-1]), Hq, Hkv, d, seed=seed)
    q, k, v = (t[0] for t in _dev(bits, "bf16"))
    tq, tk = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    o, lse = ea.attention_ex(q, k, v, causal=causal, cu_seqlens_q=tq, cu_seqlens_k=tk,
                             max_seqlen_q=int(max(lens_q)), max_seqlen_k=int(max(lens_k)), pack_gqa=pack,
                             num_splits=splits, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = attention_varlen(vals[0][0], vals[1][0], vals[2][0], cu_q, cu_k, None, causal, window=window)
    return to_f64(o), to_f64(lse), o_ref, l_ref


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 4])
def test_varlen_mixed_lengths(gpu, causal, splits):
    lens_q, _ = make_seqlens(7, 1, 300, seed=1)
    lens_k, _ = make_seqlens(7, 1, 300, seed=2)
    lens_q[2] = 0      # a sequence with no query
    lens_k[4] = 0      # a sequence with queries but no key
    o, lse, o_ref, l_ref = _varlen(gpu, lens_q, lens_k, 4, 2, 128, causal, splits, seed=5)
    assert lse.shape == (4, int(lens_q.sum()))
    _check(o, lse, o_ref, l_ref, (causal, splits))


@pytest.mark.parametrize("pack", [0, 1])
def test_long_rows_grouped_and_packed(gpu, pack):
    """From 2048 rows on the tiled kernel stores O through a buffer resource
    over each unit's rows (with the non-temporal hint): grouped heads with and
    without head packing, in a dense batch and in a packed batch of unequal
    lengths, causal and not, every row against the oracle."""
    for causal in (False, True):
        o, lse, o_ref, l_ref = _dense(gpu, 1, 2304, 2304, 8, 2, 128, causal, pack, 1, seed=21)
        _check(o, lse, o_ref, l_ref, ("dense", pack, causal))
        lens = np.array([2500, 700, 3000], dtype=np.int64)
        o, lse, o_ref, l_ref = _varlen(gpu, lens, lens, 4, 2, 128, causal, 1, pack=pack, seed=22)
        _check(o, lse, o_ref, l_ref, ("packed", pack, causal))


@pytest.mark.parametrize("d", [64, 256])
def test_varlen_equal_q_and_k_lengths(gpu, d):
    lens, _ = make_seqlens(5, 100, 400, seed=3)
    o, lse, o_ref, l_ref = _varlen(gpu, lens, lens, 2, 2, d, True, 1, pack=0, seed=6)
    _check(o, lse, o_ref, l_ref, d)


def test_decode_at_serving_size(gpu):
    # decode against an 8192-key cache: 8 sequences, 64 query heads over 8 KV
    # heads, d = 128, the heuristic's number of key ranges; every row checked
    o, lse, o_ref, l_ref = _dense(gpu, 8, 1, 8192, 64, 8, 128, True, -1, None, seed=11)
    _check(o, lse, o_ref, l_ref, "decode 8x64/8x8192")


@pytest.mark.parametrize("splits", [None, 1])
def test_decode_long_cache(gpu, splits):
    # the longest decode the benchmark times: a 32768-key cache, 8 sequences,
    # 64 query heads over 8 KV heads, d = 128; the heuristic's key ranges and
    # one range; every row checked
    o, lse, o_ref, l_ref = _dense(gpu, 8, 1, 32768, 64, 8, 128, True, -1, splits, seed=12)
    _check(o, lse, o_ref, l_ref, ("decode 8x64/8x32768", splits))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("nq,g", [(1, 1), (2, 8), (3, 5), (16, 1), (4, 4), (3, 8)])
def test_few_rows_per_kv_head(gpu, d, nq, g):
    # up to 16 query rows per KV head run the decode kernel (3 x 8 = 24 rows
    # is just past it and runs the tiled kernel)
    for causal, splits in ((False, 1), (True, 1), (True, 3)):
        o, lse, o_ref, l_ref = _dense(gpu, 2, nq, 517, 2 * g, 2, d, causal, -1, splits, seed=d + nq + g)
        _check(o, lse, o_ref, l_ref, (d, nq, g, causal, splits))


@pytest.mark.parametrize("splits", [1, 5])
def test_varlen_decode(gpu, splits):
    # one or two new tokens per sequence against caches of mixed length,
    # including an empty cache and a sequence with no new token
    lens_k, _ = make_seqlens(9, 1, 2000, seed=7)
    lens_k[3] = 0
    lens_q = np.array([1, 2, 1, 1, 0, 2, 1, 1, 2])
    o, lse, o_ref, l_ref = _varlen(gpu, lens_q, lens_k, 8, 2, 128, True, splits, seed=8)
    _check(o, lse, o_ref, l_ref, splits)


def test_decode_f16_alpha(gpu):
    o, lse, o_ref, l_ref = _dense(gpu, 3, 1, 3000, 4, 1, 128, False, -1, 4, seed=12, dtype="f16", alpha=0.05)
    _check(o, lse, o_ref, l_ref, "f16")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [(0, 0), (16, 0), (100, 50), (-1, 30), (300, -1), (31, 32)])
def test_local_window(gpu, d, window):
    for nq, nk, causal, splits in ((200, 200, False, 1), (77, 300, True, 1), (300, 77, False, 3)):
        o, lse, o_ref, l_ref = _dense(gpu, 2, nq, nk, 4, 2, d, causal, -1, splits, seed=d + nq, window=window)
        _check(o, lse, o_ref, l_ref, (d, window, nq, nk, causal, splits))


@pytest.mark.parametrize("window", [(256, 0), (0, -1), (1000, 10)])
def test_local_window_decode_and_varlen(gpu, window):
    o, lse, o_ref, l_ref = _dense(gpu, 3, 2, 2000, 16, 2, 128, True, -1, 4, seed=13, window=window)
    _check(o, lse, o_ref, l_ref, ("decode", window))
    lens_q, _ = make_seqlens(6, 1, 200, seed=4)
    lens_k, _ = make_seqlens(6, 1, 500, seed=5)
    o, lse, o_ref, l_ref = _varlen(gpu, lens_q, lens_k, 4, 4, 64, False, 2, seed=9, window=window)
    _check(o, lse, o_ref, l_ref, ("varlen", window))


def test_no_keys_with_null_key_pointers(gpu):
    # no sequence has keys: k and v are empty (null data pointers) and every
    # row gets O = 0, LSE = -inf, dense (N_k = 0) and packed (total_k = 0)
    import torch
    q = torch.randn((2, 5, 4, 64), device="cuda").to(torch.bfloat16)
    k = torch.empty((2, 0, 2, 64), device="cuda", dtype=torch.bfloat16)
    o, lse = gpu.attention_ex(q, k, k, causal=False, num_splits=1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    qp = q.reshape(10, 4, 64)
    kp = torch.empty((0, 2, 64), device="cuda", dtype=torch.bfloat16)
    cu_q = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    cu_k = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, lse = gpu.attention_ex(qp, kp, kp, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=6, max_seqlen_k=1,
                              num_splits=1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
