"""GPU tests of the FP8 path.

* attn_fp8_prepare must reproduce the CPU quantiser of the oracle bit for
  bit (codes and descales), with and without the Hadamard transform, per
  block and per tensor, on ragged N.
* attn_fwd_fp8 is compared with the float64 oracle on the unquantised
  inputs: RMSE(O) <= 3e-2, and with outliers the block + Hadamard variant
  must beat plain per-tensor FP8. A tighter check against the FP8-emulating
  reference (dequantised inputs, exact attention) bounds the kernel's own
  error (P rounded to e4m3, float32 accumulation).
"""
import math

import numpy as np
import pytest

from gpu_util import device_qkv, errors, to_f64
from oracle.attention import attention, attention_rows
from oracle.fp8 import emulated_fp8_attention, quantize
from synth_inputs import bf16_bits_to_f32, make_qkv

pytestmark = pytest.mark.gpu

OUTLIERS = {"rate": 1e-3, "factor": 10.0, "kind": "scale"}


def prep(ea, x, block_rows, hadamard, seed):
    import torch
    x8, ds = ea.fp8_prepare(x, block_rows, hadamard, seed)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), ds.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("block_rows", [128, 0])
@pytest.mark.parametrize("hadamard", [False, True])
def test_prepare_is_bit_exact(gpu, d, block_rows, hadamard):
    N = 300
    (q, _, _), _ = device_qkv(2, N, 3, d, seed=d + 1, outliers=OUTLIERS)
    x = to_f64(q).astype(np.float32)  # exact: bf16 values
    codes, desc = prep(gpu, q, block_rows, hadamard, 12345)
    ref_codes, ref_desc = quantize(x, block_rows, hadamard, 12345)
    np.testing.assert_array_equal(desc.reshape(ref_desc.shape).view(np.uint32), ref_desc.view(np.uint32))
    mism = np.count_nonzero(codes != ref_codes)
    assert mism == 0, f"{mism} of {codes.size} codes differ"


def test_prepare_full_size_bit_exact(gpu):
    (q, _, _), _ = device_qkv(2, 8192, 16, 128, seed=0, outliers=OUTLIERS)
    codes, desc = prep(gpu, q, 128, True, 0)
    x = to_f64(q).astype(np.float32)
    # the oracle quantiser is slow in Python loops; check a few heads fully
    for b, h in ((0, 0), (1, 15), (0, 7)):
        rc, rd = quantize(x[b:b + 1, :, h:h + 1, :], 128, True, 0)
        np.testing.assert_array_equal(codes[b, :, h], rc[0, :, 0])
        np.testing.assert_array_equal(desc[b, h], rd[0, 0])


def fp8_run(ea, q, k, v, block_rows, hadamard, causal, seed=0):
    import torch
    q8, sq = ea.fp8_prepare(q, block_rows, hadamard, seed)
    k8, sk = ea.fp8_prepare(k, block_rows, hadamard, seed)
    v8, sv = ea.fp8_prepare(v, block_rows, False, seed)
    o, lse = ea.attention_fp8(q8, k8, v8, sq, sk, sv, causal=causal, block_rows=block_rows)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 300, 777])
def test_fp8_forward_small_shapes(gpu, d, causal, N):
    (q, k, v), (qf, kf, vf) = device_qkv(2, N, 2, d, seed=N + d, outliers=OUTLIERS)
    o, lse = fp8_run(gpu, q, k, v, 128, True, causal)
    o_ref, l_ref = attention(qf, kf, vf, 1 / math.sqrt(d), causal)
    err = errors(o, o_ref, lse, l_ref)
    print((d, causal, N), err)
    assert err["rmse"] <= 3e-2, err
    assert np.isfinite(o).all()


@pytest.mark.parametrize("hadamard,block_rows", [(True, 128), (False, 0), (False, 128), (True, 0)])
def test_fp8_forward_tracks_emulated_reference(gpu, hadamard, block_rows):
    """Kernel vs. exact attention on the dequantised inputs: isolates the
    kernel's own error (P in e4m3, float32 sums) from input quantisation."""
    d, N = 128, 500
    (q, k, v), (qf, kf, vf) = device_qkv(1, N, 2, d, seed=21, outliers=OUTLIERS)
    o, lse = fp8_run(gpu, q, k, v, block_rows, hadamard, True, seed=3)
    # the oracle's own quantisation of the same bf16 inputs (the GPU prepare
    # matches it bit for bit, which the test_prepare_* tests check)
    o_emu, l_emu = emulated_fp8_attention(qf, kf, vf, 1 / math.sqrt(d), True, block_rows, hadamard, 3)
    err = errors(o, o_emu, lse, l_emu)
    print("vs emulated", hadamard, block_rows, err)
    assert err["rmse"] <= 1e-2, err
    # Scores come from e4m3 products accumulated by the fp8 MFMA; the pages
    # warn that FP8 tensor-core accumulation can be narrower than float32
    # ("FlashAttention-3 on Hopper", section 6.1). With per-tensor scales and
    # x10 outliers the scores reach ~20 and LSE deviates by up to ~2.3e-3.
    assert err["lse_abs"] <= 5e-3, err


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [64, 150, 200, 300])
def test_fp8_every_tail_tracks_emulated_reference(gpu, d, causal, N):
    """One, three, four and five 64-key tiles per query block: the kernel
    walks tiles in pairs and ends in one of three tails, and every output
    dimension of every tail must track exact attention on the dequantised
    inputs (a lost product shows up as one column far off, which the
    whole-tensor RMSE would average away)."""
    (q, k, v), (qf, kf, vf) = device_qkv(1, N, 2, d, seed=5 + N + d)
    o, lse = fp8_run(gpu, q, k, v, 128, True, causal, seed=7)
    o_emu, l_emu = emulated_fp8_attention(qf, kf, vf, 1 / math.sqrt(d), causal, 128, True, 7)
    err = errors(o, o_emu, lse, l_emu)
    col = np.sqrt(np.mean((o - o_emu) ** 2, axis=(0, 1)))  # per (head, dim)
    print((d, causal, N), err, "worst column rmse", float(col.max()))
    assert err["rmse"] <= 1e-2, err
    assert col.max() <= 2e-2, (err, float(col.max()))
    assert err["lse_abs"] <= 5e-3, err


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 1), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_rows", [128, 0])
def test_fp8_grouped_heads(gpu, hq, hkv, causal, block_rows):
    """attn_fwd_fp8_ex: query head h reads key/value head h / (Hq / Hkv).
    Against exact grouped attention on the oracle's own dequantised inputs
    (the kernel's share) and on the unquantised inputs (the FP8 bound)."""
    import torch
    from oracle.fp8 import dequantize
    from oracle.variants import attention_gqa
    from synth_inputs import make_qkv_gqa
    B, N, d = 2, 300, 128
    bits, (qf, kf, vf) = make_qkv_gqa(B, N, N, hq, hkv, d, seed=hq * 10 + hkv)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
    q8, sq = gpu.fp8_prepare(q, block_rows, True, 7)
    k8, sk = gpu.fp8_prepare(k, block_rows, True, 7)
    v8, sv = gpu.fp8_prepare(v, block_rows, False, 7)
    o, lse = gpu.attention_fp8(q8, k8, v8, sq, sk, sv, causal=causal, block_rows=block_rows)
    torch.cuda.synchronize()
    o, lse = to_f64(o), lse.cpu().numpy().astype(np.float64)
    deq = [dequantize(*quantize(x, block_rows, had, 7), block_rows)
           for x, had in ((qf, True), (kf, True), (vf, False))]
    o_emu, l_emu = attention_gqa(deq[0], deq[1], deq[2], 1 / math.sqrt(d), causal)
    o_ref, l_ref = attention_gqa(qf, kf, vf, 1 / math.sqrt(d), causal)
    err_emu = errors(o, o_emu, lse, l_emu)
    err = errors(o, o_ref, lse, l_ref)
    print((hq, hkv, causal, block_rows), err_emu, err)
    assert err_emu["rmse"] <= 1e-2 and err_emu["lse_abs"] <= 5e-3, err_emu
    assert err["rmse"] <= 3e-2, err


def test_fp8_rmse_and_hadamard_beats_per_tensor_with_outliers(gpu):
    """The FP8 configuration of the benchmark: H=16, d=128, N in 1k..16k,
    B = 16k/N, N(0,1) inputs with 0.1% of entries scaled by 10, 128-row block
    scales with and without the Hadamard transform, and per-tensor scales.
    Compared on sampled rows of a few heads against the oracle on the
    unquantised inputs."""
    import torch
    rng = np.random.default_rng(0)
    for N in (1024, 2048, 4096, 8192, 16384):
        B, H, d = 16384 // N, 16, 128
        (q, k, v), (qf, kf, vf) = device_qkv(B, N, H, d, seed=N, outliers=OUTLIERS)
        pairs = [(0, 0), (B - 1, H - 1), (B // 2, 5)]
        samples = [(b, h, np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 40)]))) for b, h in pairs]
        refs = attention_rows(qf, kf, vf, 1 / math.sqrt(d), False, samples)
        orf = np.concatenate([r[0] for r in refs])
        res = {}
        for name, had, br in (("block+hadamard", True, 128), ("per-tensor", False, 0)):
            o, lse = fp8_run(gpu, q, k, v, br, had, False)
            og = np.concatenate([o[b, rows, h] for b, h, rows in samples])
            res[name] = math.sqrt(np.mean((og - orf) ** 2))
            assert np.isfinite(o).all()
        print(N, res, flush=True)
        assert res["block+hadamard"] <= 3e-2, (N, res)
        assert res["block+hadamard"] < res["per-tensor"], (N, res)


@pytest.mark.parametrize("N", [1024, 2048, 4096, 8192, 16384])
def test_fp8_block_scales_without_hadamard(gpu, N):
    """The configuration's other variant: 128-row block scales without the
    transform, on the same outlier inputs and shapes (B = 16k/N, H = 16,
    d = 128). Its error is set by quantising the inputs: an x10 outlier
    sets the scale of its whole 128-row block. So besides the unquantised
    oracle it is compared with the oracle's own e4m3 quantisation of the same
    inputs (exact attention on the dequantised tensors, on the same rows):
    the kernel may add at most 5e-3 to that, and it must meet 3e-2 wherever
    the quantised inputs alone leave at least 5e-3 of room. (At N = 16384
    they alone are 0.030 from exact attention over the whole tensor.)"""
    from oracle.fp8 import dequantize
    B, H, d = 16384 // N, 16, 128
    (q, k, v), (qf, kf, vf) = device_qkv(B, N, H, d, seed=N, outliers=OUTLIERS)
    rng = np.random.default_rng(N)
    samples = [(b, h, np.unique(np.concatenate([[0, 1, N - 1], rng.integers(0, N, 40)])))
               for b, h in ((0, 0), (B - 1, H - 1), (B // 2, 5))]
    alpha = 1 / math.sqrt(d)
    orf = np.concatenate([r[0] for r in attention_rows(qf, kf, vf, alpha, False, samples)])
    deq = [dequantize(*quantize(x, 128, False, 0), 128) for x in (qf, kf, vf)]
    oem = np.concatenate([r[0] for r in attention_rows(deq[0], deq[1], deq[2], alpha, False, samples)])
    o, _ = fp8_run(gpu, q, k, v, 128, False, False)
    assert np.isfinite(o).all()
    og = np.concatenate([o[b, rows, h] for b, h, rows in samples])
    rmse = math.sqrt(np.mean((og - orf) ** 2))
    quant_only = math.sqrt(np.mean((oem - orf) ** 2))
    kernel_share = math.sqrt(np.mean((og - oem) ** 2))
    print(N, {"block": rmse, "quantised inputs alone": quant_only, "kernel vs quantised": kernel_share}, flush=True)
    assert rmse <= quant_only + 5e-3, (N, rmse, quant_only)
    assert kernel_share <= 1e-2, (N, kernel_share)
    if quant_only <= 2.5e-2:
        assert rmse <= 3e-2, (N, rmse, quant_only)


@pytest.mark.parametrize("d,H", [(64, 32), (128, 16), (256, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_full_size_sampled(gpu, d, H, causal):
    """Every head dimension at N = 8192 (B = 2, 16k tokens, hidden 2048), both
    masks, with the outlier inputs and 128-row blocks + Hadamard: sampled rows
    (first, last and random, so the causal rows see 1 to 8192 keys) against
    the oracle on the unquantised inputs."""
    N, B = 8192, 2
    (q, k, v), (qf, kf, vf) = device_qkv(B, N, H, d, seed=31 + d, outliers=OUTLIERS)
    rng = np.random.default_rng(d)
    samples = [(b, h, np.unique(np.concatenate([[0, 1, 63, 64, N - 1], rng.integers(0, N, 30)])))
               for b, h in ((0, 0), (B - 1, H - 1))]
    o, lse = fp8_run(gpu, q, k, v, 128, True, causal)
    refs = attention_rows(qf, kf, vf, 1 / math.sqrt(d), causal, samples)
    og = np.concatenate([o[b, rows, h] for b, h, rows in samples])
    lg = np.concatenate([lse[b, h, rows] for b, h, rows in samples])
    orf = np.concatenate([r[0] for r in refs])
    lrf = np.concatenate([r[1] for r in refs])
    err = errors(og, orf, lg, lrf)
    print((d, causal), err)
    assert np.isfinite(o).all()
    assert err["rmse"] <= 3e-2, err


def test_fp8_hadamard_beats_per_tensor_on_full_heads(gpu):
    """The ordering of the outlier benchmark on every row of 8 whole heads
    (N = 2048, B = 8, H = 16, d = 128): a sample of ~130 rows gives a noisy
    RMSE (it put per-tensor within 15% of block + Hadamard where the full rows
    differ by about 2x), so this measures all 16k rows."""
    N, B, H, d = 2048, 8, 16, 128
    (q, k, v), (qf, kf, vf) = device_qkv(B, N, H, d, seed=N, outliers=OUTLIERS)
    heads = [(i, (5 * i) % H) for i in range(B)]
    refs = attention_rows(qf, kf, vf, 1 / math.sqrt(d), False, [(b, h, np.arange(N)) for b, h in heads])
    orf = np.concatenate([r[0] for r in refs])
    res = {}
    for name, had, br in (("block+hadamard", True, 128), ("per-tensor", False, 0)):
        o, _ = fp8_run(gpu, q, k, v, br, had, False)
        og = np.concatenate([o[b, :, h] for b, h in heads])
        assert np.isfinite(og).all(), name
        res[name] = math.sqrt(np.mean((og - orf) ** 2))
    print(res, flush=True)
    assert res["block+hadamard"] <= 3e-2, res
    assert res["block+hadamard"] < 0.75 * res["per-tensor"], res


def test_fp8_tensors_past_two_billion_elements(gpu):
    """Prepare and forward on tensors of 17 x 65536 x 16 x 128 = 2.28e9
    elements (the last batch entries start past element 2^31): the codes of
    sampled rows of the last entry equal the oracle's quantiser on the same
    bf16 rows, and sampled outputs stay within the FP8 bound of the fp64
    oracle on the unquantised inputs. Inputs come from a seeded torch
    generator on the device."""
    import torch
    from oracle.attention import attention_head
    B, N, H, d = 17, 65536, 16, 128
    g = torch.Generator(device="cuda").manual_seed(23)
    q, k, v = [torch.randn((B, N, H, d), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3)]
    q8, sq = gpu.fp8_prepare(q, 128, True, 5)
    k8, sk = gpu.fp8_prepare(k, 128, True, 5)
    v8, sv = gpu.fp8_prepare(v, 128, False, 5)
    o, lse = gpu.attention_fp8(q8, k8, v8, sq, sk, sv, causal=True, block_rows=128)
    torch.cuda.synchronize()
    # codes of one 128-row block of the last batch entry, head 15, bit for bit
    b, h, blk = 16, 15, 511
    rows = slice(128 * blk, 128 * blk + 128)
    xk = k[b, rows, h].float().cpu().numpy()[None, :, None, :]
    codes, desc = quantize(xk, 128, True, 5)
    got = k8[b, rows, h].cpu().numpy()
    assert np.array_equal(got, codes[0, :, 0, :])
    assert float(sk[b, h, blk].cpu()) == float(desc[0, 0, 0])
    rng = np.random.default_rng(23)
    for b, h in ((0, 0), (16, 15)):
        sel = np.array(sorted({1, 40000, N - 1} | set(rng.integers(1, N, 12).tolist())))
        qf = q[b, :, h].float().cpu().numpy().astype(np.float64)
        kf = k[b, :, h].float().cpu().numpy().astype(np.float64)
        vf = v[b, :, h].float().cpu().numpy().astype(np.float64)
        o_ref, l_ref = attention_head(qf, kf, vf, 1 / math.sqrt(d), True, rows=sel)
        og = o[b, sel, h].float().cpu().numpy().astype(np.float64)
        err = errors(og, o_ref)
        print((b, h), err, flush=True)
        assert err["rmse"] <= 3e-2, err
    del q, k, v, q8, k8, v8, o, lse
    torch.cuda.empty_cache()
