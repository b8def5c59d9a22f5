"""attn_fwd_ex_noalloc against attn_fwd_ex (GPU).

The allocation-free entry point runs the same kernels with the split-KV
range states in the library's static per-GPU array instead of a caller
workspace, so its outputs must equal attn_fwd_ex's bit for bit. Two calls in
a row, the second with a smaller input, check that the array's leftover
contents from the first call do not leak into the second. The tiled kernel
(many query rows) and the decode kernel (one query row per sequence, grouped
heads) are both covered, as is a packed batch.
"""
import numpy as np
import pytest

from gpu_util import device_qkv
from synth_inputs import make_qkv_gqa

pytestmark = pytest.mark.gpu


def _gqa(B, Nq, Nk, Hq, Hkv, d, seed):
    import torch
    bits, _ = make_qkv_gqa(B, Nq, Nk, Hq, Hkv, d, seed=seed)
    return [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda() for b in bits]


def _both(ea, q, k, v, causal, num_splits, **kw):
    """(o, lse) of attn_fwd_ex with a torch workspace and of attn_fwd_ex_noalloc."""
    import torch
    o_ref = torch.empty_like(q)
    lse_shape = kw.pop("lse_shape")
    lse_ref = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    total_q = q.shape[0] if q.dim() == 3 else q.shape[0] * q.shape[1]
    nb = ea.attn_splitkv_workspace_bytes(num_splits, total_q, q.shape[-2], q.shape[-1])
    ws = torch.empty(max(nb // 4, 4), dtype=torch.float32, device=q.device)
    ea.attn_fwd_ex(q, k, v, o_ref, lse_ref, causal=causal, num_splits=num_splits, workspace=ws, **kw)
    # outputs start as NaN so a row the call fails to write shows up
    o = torch.full_like(q, float("nan"))
    lse = torch.full(lse_shape, float("nan"), dtype=torch.float32, device=q.device)
    ea.attn_fwd_ex_noalloc(q, k, v, o, lse, causal=causal, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return (o_ref, lse_ref), (o, lse)


def _assert_identical(ref, got, tag):
    import torch
    (o_ref, l_ref), (o, l) = ref, got
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), tag
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32)), tag


def test_noalloc_matches_workspace_call_twice_tiled(gpu):
    # tiled kernel: 300 query rows against 2000 keys in 4 ranges, then a
    # smaller problem (fewer rows, heads, keys and ranges) on the same array
    for i, (B, Nq, Nk, Hq, Hkv, d, splits, causal) in enumerate(
            ((2, 300, 2000, 8, 2, 128, 4, True), (1, 130, 700, 4, 4, 64, 3, False))):
        q, k, v = _gqa(B, Nq, Nk, Hq, Hkv, d, seed=40 + i)
        print("tiled call", i, (B, Nq, Nk, Hq, Hkv, d, splits, causal), flush=True)
        ref, got = _both(gpu, q, k, v, causal, splits, lse_shape=(B, Hq, Nq))
        _assert_identical(ref, got, ("tiled", i))


def test_noalloc_matches_workspace_call_twice_decode(gpu):
    # decode kernel (one query row, 8 query heads over 2 KV heads): 8 ranges
    # over a 4096-key cache, then 2 ranges over 1000 keys with fewer sequences
    for i, (B, Nk, splits) in enumerate(((4, 4096, 8), (2, 1000, 2))):
        q, k, v = _gqa(B, 1, Nk, 8, 2, 128, seed=50 + i)
        print("decode call", i, (B, Nk, splits), flush=True)
        ref, got = _both(gpu, q, k, v, True, splits, lse_shape=(B, 8, 1))
        _assert_identical(ref, got, ("decode", i))


def test_noalloc_packed_batch_and_one_range(gpu):
    import torch
    # packed batch of three sequences (one without keys) in 3 ranges, then a
    # call with one range, which uses no workspace at all
    lens_q, lens_k = [100, 37, 5], [500, 0, 260]
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32, device="cuda")
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32, device="cuda")
    (q, _, _), _ = device_qkv(1, sum(lens_q), 4, 128, seed=61)
    (k, v, _), _ = device_qkv(1, sum(lens_k), 2, 128, seed=62)
    q, k, v = q[0].contiguous(), k[0].contiguous(), v[0].contiguous()
    kw = dict(cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=max(lens_q), max_seqlen_k=max(lens_k),
              lse_shape=(4, sum(lens_q)))
    print("packed call", flush=True)
    ref, got = _both(gpu, q, k, v, True, 3, **dict(kw))
    _assert_identical(ref, got, "packed")
    (q1, k1, v1), _ = device_qkv(2, 200, 2, 128, seed=63)
    print("one-range call", flush=True)
    ref, got = _both(gpu, q1, k1, v1, False, 1, lse_shape=(2, 2, 200))
    _assert_identical(ref, got, "one range")


def test_noalloc_rejects_oversized_split_state(gpu):
    import torch
    # 128 ranges of 64 query rows x 32 heads x d=256 need 269 MB: rejected
    # before any launch, outputs untouched
    q = torch.zeros((1, 64, 32, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8192, 32, 256), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.zeros((1, 32, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu.AttnError, match="static"):
        gpu.attn_fwd_ex_noalloc(q, k, k, o, lse, num_splits=128)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
