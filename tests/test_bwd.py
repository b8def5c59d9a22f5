"""GPU parity of the 16-bit backward (attn_bwd) against the float64 oracle.

Inputs: Q, K, V from ``synth_inputs.make_qkv`` and dO from ``make_dout``
(N(0,1) rounded to bf16); O and LSE come from the library's own forward, as a
training step would pass them. The oracle recomputes everything in float64
from the same rounded Q, K, V, dO.

Tolerances (derived from the arithmetic: P, dS and the outputs are rounded to
16 bits, 2^-9 relative each; sums are float32; D is formed from the 16-bit
O): per gradient, max |g - g_ref| <= 2e-2 * max |g_ref| and
rms(g - g_ref) <= 1e-2 * rms(g_ref).
"""
import math

import numpy as np
import pytest

from gpu_util import device_qkv, to_f64
from oracle.attention_bwd import attention_backward
from synth_inputs import make_dout

REL_MAX = 2e-2
REL_RMS = 1e-2

pytestmark = pytest.mark.gpu


def _run(ea, B, N, H, d, causal, seed=0, dtype="bf16", alpha=None):
    import torch
    (q, k, v), vals = device_qkv(B, N, H, d, seed=seed, dtype=dtype)
    bits, do_vals = make_dout(B, N, H, d, seed=seed, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    do = torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    o, lse = ea.attention(q, k, v, causal=causal, alpha=alpha)
    dq, dk, dv = ea.attention_backward(q, k, v, o, lse, do, causal=causal, alpha=alpha)
    torch.cuda.synchronize()
    return (dq, dk, dv), vals, do_vals, (q, k, v, o, lse, do)


def _rel(g, ref):
    scale_max = float(np.abs(ref).max()) or 1.0
    scale_rms = float(math.sqrt(np.mean(ref ** 2))) or 1.0
    diff = g - ref
    return {"rel_max": float(np.abs(diff).max()) / scale_max,
            "rel_rms": float(math.sqrt(np.mean(diff ** 2))) / scale_rms}


def _check(grads, vals, do_vals, causal, alpha=None, tag=""):
    refs = attention_backward(*vals, do_vals, alpha, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        e = _rel(to_f64(g), r)
        assert np.isfinite(to_f64(g)).all(), (tag, name)
        assert e["rel_max"] <= REL_MAX and e["rel_rms"] <= REL_RMS, (tag, name, e)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 129, 300])
def test_bwd_small_shapes(gpu, d, causal, N):
    grads, vals, do_vals, _ = _run(gpu, 2, N, 2, d, causal, seed=N)
    _check(grads, vals, do_vals, causal, tag=(d, causal, N))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_several_tiles(gpu, causal):
    # 1024 queries and keys: 8 key blocks of 128, 32 query tiles of 32
    grads, vals, do_vals, _ = _run(gpu, 1, 1024, 2, 128, causal, seed=5)
    _check(grads, vals, do_vals, causal, tag=("n1024", causal))


def test_bwd_f16_and_alpha(gpu):
    grads, vals, do_vals, _ = _run(gpu, 1, 200, 2, 64, True, seed=7, dtype="f16", alpha=0.3)
    _check(grads, vals, do_vals, True, alpha=0.3, tag="f16")


def test_bwd_delta_is_rowsum_of_dout_times_o(gpu):
    # the backward is handed the oracle's O (rounded to bf16), so the
    # expected D = rowsum(dO o O) depends on nothing the GPU computed
    import torch
    from oracle.attention import attention
    from synth_inputs import bf16_bits_to_f32, f32_to_bf16_bits
    _, vals, do_vals, (q, k, v, _, lse, do) = _run(gpu, 1, 77, 3, 64, False, seed=9)
    B, N, H, d = q.shape
    o_ref, _ = attention(*vals, 1 / math.sqrt(d), False)
    obits = f32_to_bf16_bits(o_ref.astype(np.float32))
    o_in = torch.from_numpy(obits.view(np.int16)).view(torch.bfloat16).cuda()
    delta = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gpu.attn_bwd(q, k, v, o_in, do, lse, dq, dk, dv, delta)
    torch.cuda.synchronize()
    ref = np.einsum("bnhd,bnhd->bhn", do_vals, bf16_bits_to_f32(obits).astype(np.float64))
    np.testing.assert_allclose(to_f64(delta), ref, rtol=1e-5, atol=1e-5)


def test_bwd_is_deterministic(gpu):
    import torch
    g1, _, _, t = _run(gpu, 1, 300, 2, 128, True, seed=11)
    q, k, v, o, lse, do = t
    g2 = gpu.attention_backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_head_dim_256_several_tiles(gpu, causal):
    # d = 256 runs the dK/dV kernel twice (dV, then dK)
    grads, vals, do_vals, _ = _run(gpu, 1, 700, 2, 256, causal, seed=13)
    _check(grads, vals, do_vals, causal, tag=("d256", causal))


def _run_gqa(ea, B, Nq, Nk, Hq, Hkv, d, causal, seed=0):
    import torch
    from synth_inputs import make_qkv_gqa
    bits, vals = make_qkv_gqa(B, Nq, Nk, Hq, Hkv, d, seed=seed)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
    dbits, dvals = make_dout(B, Nq, Hq, d, seed=seed)
    do = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
    o, lse = ea.attention_ex(q, k, v, causal=causal, pack_gqa=0, num_splits=1)
    grads = ea.attention_backward_ex(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    return grads, vals, dvals


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (6, 1), (3, 3)])
def test_bwd_grouped_heads(gpu, d, hq, hkv):
    from oracle.attention_bwd import attention_backward_gqa
    for nq, nk, causal in ((150, 150, False), (77, 300, True), (300, 77, True), (200, 130, False)):
        grads, vals, dvals = _run_gqa(gpu, 2, nq, nk, hq, hkv, d, causal, seed=d + hq + nq)
        refs = attention_backward_gqa(*vals, dvals, None, causal)
        for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
            e = _rel(to_f64(g), r)
            assert np.isfinite(to_f64(g)).all(), (d, hq, hkv, nq, nk, name)
            assert e["rel_max"] <= REL_MAX and e["rel_rms"] <= REL_RMS, (d, hq, hkv, nq, nk, causal, name, e)


def test_bwd_grouped_heads_deterministic_and_empty_queries(gpu):
    import torch
    grads1, _, _ = _run_gqa(gpu, 1, 257, 513, 8, 2, 128, True, seed=3)
    grads2, _, _ = _run_gqa(gpu, 1, 257, 513, 8, 2, 128, True, seed=3)
    for a, b in zip(grads1, grads2):
        assert torch.equal(a, b)
    # keys that no query sees (causal, N_q < N_k: keys past the last query's
    # diagonal do not exist; the first N_k - N_q keys are seen by every row)
    # and N_q = 0: dK = dV = 0
    k = torch.randn((1, 64, 2, 64), device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 64, 2, 64), device="cuda").to(torch.bfloat16)
    q = torch.empty((1, 0, 4, 64), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((1, 4, 0), device="cuda", dtype=torch.float32)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    gpu.attn_bwd_ex(q, k, v, q, q, lse, torch.empty_like(q), dk, dv, torch.empty_like(lse), causal=False)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def _blind(nq, nk, causal, win):
    """Queries that see no key and keys that no query sees, from the mask."""
    from oracle.attention import causal_mask
    from oracle.variants import window_mask
    hidden = window_mask(nq, nk, *win)
    if causal:
        hidden = hidden | causal_mask(nq, nk)
    return hidden.all(axis=1), hidden.all(axis=0)


def _grads_ok(grads, refs, tag, blind=None):
    """Tolerances on dq, dk, dv; with ``blind`` = (rows, keys) boolean masks
    over the sequence axis (axis -3), those rows of dq and keys of dk, dv are
    exactly zero."""
    for i, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), grads, refs)):
        gv = to_f64(g)
        assert np.isfinite(gv).all(), (tag, name)
        e = _rel(gv, r)
        assert e["rel_max"] <= REL_MAX and e["rel_rms"] <= REL_RMS, (tag, name, e)
        if blind is not None:
            m = blind[0] if i == 0 else blind[1]
            assert np.all(np.take(gv, np.nonzero(m)[0], axis=-3) == 0), (tag, name)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bwd_local_windows(gpu, d):
    # sliding windows of the forward (left, right), with and without causal,
    # on N_q != N_k and grouped heads; every window leaves some keys or rows
    # outside the band, and (0, 0) a single diagonal
    import torch
    from oracle.attention_bwd import attention_backward_gqa
    from synth_inputs import make_qkv_gqa
    cases = [(300, 300, True, (40, -1)), (200, 333, True, (100, -1)), (333, 200, False, (17, 25)),
             (260, 260, False, (2, 1)), (150, 400, False, (-1, 30)), (400, 150, False, (64, -1)),
             (129, 500, True, (60, -1))]
    for i, (nq, nk, causal, win) in enumerate(cases):
        bits, vals = make_qkv_gqa(2, nq, nk, 4, 2, d, seed=d + i)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
        dbits, dvals = make_dout(2, nq, 4, d, seed=d + i)
        do = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).cuda()
        o, lse = gpu.attention_ex(q, k, v, causal=causal, pack_gqa=0, num_splits=1, window=win)
        grads = gpu.attention_backward_ex(q, k, v, o, lse, do, causal=causal, window=win)
        torch.cuda.synchronize()
        refs = attention_backward_gqa(*vals, dvals, None, causal, window=win)
        _grads_ok(grads, refs, (d, nq, nk, causal, win), _blind(nq, nk, causal, win))


def _run_varlen(ea, lens_q, lens_k, Hq, Hkv, d, causal, window=(-1, -1), seed=0, dtype="bf16", alpha=None):
    import torch
    from oracle.attention_bwd import attention_backward_varlen
    from synth_inputs import make_qkv_gqa
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    tq_, tk_ = int(cu_q[-1]), int(cu_k[-1])
    bits, vals = make_qkv_gqa(1, tq_, tk_, Hq, Hkv, d, seed=seed, dtype=dtype)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(b[0]).view(np.int16)).view(tdt).cuda() for b in bits)
    dbits, dvals = make_dout(1, tq_, Hq, d, seed=seed, dtype=dtype)
    do = torch.from_numpy(np.ascontiguousarray(dbits[0]).view(np.int16)).view(tdt).cuda()
    tq, tk = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    kw = dict(cu_seqlens_q=tq, cu_seqlens_k=tk, max_seqlen_q=int(max(lens_q)), max_seqlen_k=int(max(lens_k)),
              window=window)
    o, lse = ea.attention_ex(q, k, v, causal=causal, alpha=alpha, pack_gqa=0, num_splits=1, **kw)
    grads = ea.attention_backward_ex(q, k, v, o, lse, do, causal=causal, alpha=alpha, **kw)
    torch.cuda.synchronize()
    refs = attention_backward_varlen(vals[0][0], vals[1][0], vals[2][0], dvals[0], cu_q, cu_k, alpha, causal, window)
    # rows and keys of each sequence that the mask leaves out, over the packed axis
    rows, keys = [], []
    for lq, lk in zip(lens_q, lens_k):
        r, c = _blind(int(lq), int(lk), causal, window)
        rows.append(r if lk > 0 else np.ones(int(lq), dtype=bool))
        keys.append(c if lq > 0 else np.ones(int(lk), dtype=bool))
    blind = (np.concatenate(rows + [np.zeros(0, bool)]), np.concatenate(keys + [np.zeros(0, bool)]))
    return grads, refs, blind


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_mixed_lengths(gpu, causal):
    from synth_inputs import make_seqlens
    lens_q, _ = make_seqlens(7, 1, 300, seed=1)
    lens_k, _ = make_seqlens(7, 1, 300, seed=2)
    lens_q[2] = 0      # a sequence with no query: its dK, dV are zero
    lens_k[4] = 0      # a sequence with queries but no key: its dQ is zero
    grads, refs, blind = _run_varlen(gpu, lens_q, lens_k, 4, 2, 128, causal, seed=5)
    assert blind[0].any() and blind[1].any()
    _grads_ok(grads, refs, ("varlen", causal), blind)


@pytest.mark.parametrize("d", [64, 256])
def test_bwd_varlen_equal_lengths_and_windows(gpu, d):
    from synth_inputs import make_seqlens
    lens, _ = make_seqlens(5, 100, 400, seed=3)
    for causal, win in ((True, (-1, -1)), (True, (50, -1)), (False, (20, 20))):
        grads, refs, blind = _run_varlen(gpu, lens, lens, 2, 2, d, causal, win, seed=6 + d)
        _grads_ok(grads, refs, ("varlen", d, causal, win), blind)


def test_bwd_varlen_matches_dense_bitwise(gpu):
    # one packed sequence is the dense problem: same kernels, same bits
    import torch
    lens = np.array([333], dtype=np.int64)
    grads_v, _, _ = _run_varlen(gpu, lens, lens, 4, 2, 128, True, seed=9)
    grads_d, _, _ = _run_gqa(gpu, 1, 333, 333, 4, 2, 128, True, seed=9)
    for a, b in zip(grads_v, grads_d):
        assert torch.equal(a, b[0])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,H", [(64, 32), (128, 16), (256, 8)])
def test_bwd_full_size_sampled(gpu, causal, d, H):
    # the 16k-token shapes at every head dimension (B=2, N=8192, hidden 2048;
    # d=128 is the call bench.py times): dQ at 48 query rows and dK, dV at 48
    # keys (the edges of the first two 128-blocks, the last row and key,
    # random others) of two heads, against the oracle evaluated row by row
    from oracle.attention_bwd import attention_backward_sampled
    B, N = 2, 8192
    grads, vals, do_vals, _ = _run(gpu, B, N, H, d, causal, seed=0)
    dq, dk, dv = (to_f64(g) for g in grads)
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([[0, 1, 127, 128, 255, N - 1], rng.integers(0, N, 42)]))
    for b, h in ((0, 3), (1, H - 2)):
        q, k, v = (x[b, :, h] for x in vals)
        refs = attention_backward_sampled(q, k, v, do_vals[b, :, h], 1.0 / math.sqrt(d), causal, idx, idx)
        for name, g, r in zip(("dq", "dk", "dv"), (dq[b, idx, h], dk[b, idx, h], dv[b, idx, h]), refs):
            assert np.isfinite(g).all(), (b, h, name)
            e = _rel(g, r)
            assert e["rel_max"] <= REL_MAX and e["rel_rms"] <= REL_RMS, (causal, b, h, name, e)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bwd_f16_grouped_varlen_window_alpha(gpu, d):
    # f16 inputs, 6 query heads over 2 KV heads, packed sequences of unequal
    # query and key lengths, a causal sliding window and a non-default alpha,
    # all in one call
    from synth_inputs import make_seqlens
    lens_q, _ = make_seqlens(4, 30, 260, seed=20 + d)
    lens_k, _ = make_seqlens(4, 30, 260, seed=30 + d)
    grads, refs, blind = _run_varlen(gpu, lens_q, lens_k, 6, 2, d, True, (70, -1), seed=40 + d, dtype="f16",
                                     alpha=0.2)
    _grads_ok(grads, refs, ("f16", d), blind)
