"""Pins for the FP8 part of the oracle: Hadamard transform, sign generator,
e4m3 encoding and block quantisation."""
import math

import numpy as np
import pytest

from oracle.attention import attention
from oracle.fp8 import (E4M3_MAX, dequantize, e4m3_decode, e4m3_encode, emulated_fp8_attention, fwht,
                        hadamard_matrix, hadamard_signs, quantize, splitmix64, sylvester)
from synth_inputs import make_qkv, make_qkv_f32

GOLDEN = 0x9E3779B97F4A7C15


def test_splitmix64_published_outputs():
    # A SplitMix64 generator seeded with state 0 yields these first three
    # outputs (reference implementation accompanying Steele, Lea and Flood,
    # OOPSLA 2014). splitmix64(x) is the first output from state x, so the
    # k-th output from state 0 is splitmix64((k - 1) * golden).
    assert splitmix64(0) == 0xE220A8397B1DCDAF
    assert splitmix64(GOLDEN) == 0x6E789E6AA1B965F4
    assert splitmix64((2 * GOLDEN) & ((1 << 64) - 1)) == 0x06C45D188009454F


def test_hadamard_signs_are_pm1_balanced_and_seeded():
    s = hadamard_signs(4096, 0)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 0.06
    assert not np.array_equal(hadamard_signs(128, 0), hadamard_signs(128, 1))
    np.testing.assert_array_equal(hadamard_signs(128, 7), hadamard_signs(256, 7)[:128])


@pytest.mark.parametrize("d", [1, 2, 4, 64, 128, 256])
def test_sylvester_is_hadamard(d):
    h = sylvester(d)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))
    assert set(np.unique(h)) <= {-1.0, 1.0}
    np.testing.assert_array_equal(h, h.T)
    if d >= 2:
        np.testing.assert_array_equal(sylvester(2), [[1, 1], [1, -1]])
        top = sylvester(d // 2)
        np.testing.assert_array_equal(h[: d // 2, d // 2:], top)
        np.testing.assert_array_equal(h[d // 2:, d // 2:], -top)


def test_sylvester_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        sylvester(96)


@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_fwht_equals_explicit_product(d):
    x = np.random.default_rng(d).standard_normal((5, 3, d))
    np.testing.assert_allclose(fwht(x, np.float64), x @ sylvester(d), atol=1e-12)
    # float32 path stays within float32 rounding of the exact product
    y32 = fwht(x.astype(np.float32), np.float32)
    np.testing.assert_allclose(y32, x @ sylvester(d), atol=1e-4 * math.sqrt(d))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_hadamard_matrix_is_orthogonal_and_preserves_attention(d):
    m = hadamard_matrix(d, 3)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-12)
    _, (q, k, v) = make_qkv(1, 40, 2, d, seed=4)
    o1, l1 = attention(q, k, v, causal=True)
    o2, l2 = attention(q @ m, k @ m, v, causal=True)
    np.testing.assert_allclose(o2, o1, atol=1e-10)
    np.testing.assert_allclose(l2, l1, atol=1e-10)


def test_e4m3_known_codes():
    # OCP 8-bit floating point specification (OFP8, 2023), E4M3 format:
    # bias 7, max normal 448 = S.1111.110, min normal 2^-6, min subnormal
    # 2^-9, NaN = S.1111.111, no infinities.
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x44: 3.0, 0xC0: -2.0, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x77: 240.0}
    for c, val in table.items():
        assert e4m3_decode(np.array([c], np.uint8))[0] == val
        assert e4m3_encode(np.array([val], np.float32))[0] == c
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_rounding_is_nearest_even_and_saturating():
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.0624, 0x38), (1.0626, 0x39),
             (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (2.0 ** -10 * 1.0001, 0x01), (15 * 2.0 ** -10, 0x08)]
    for x, c in cases:
        assert e4m3_encode(np.array([x], np.float32))[0] == c, (x, hex(c))


def test_e4m3_round_trip_all_finite_codes_and_monotone():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert fin.sum() == 254
    back = e4m3_encode(vals[fin].astype(np.float32))
    np.testing.assert_array_equal(back, codes[fin])
    pos = np.sort(vals[(codes < 0x80) & fin])
    assert np.all(np.diff(pos) > 0) and pos[-1] == E4M3_MAX


def test_e4m3_encode_matches_torch_float8_cast_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 120)]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(x), ref)


def test_e4m3_relative_error_bound_in_normal_range():
    x = np.random.default_rng(10).uniform(2.0 ** -6, 448, 100000).astype(np.float32)
    err = np.abs(e4m3_decode(e4m3_encode(x)) - x) / x
    assert err.max() <= 2.0 ** -4 + 1e-12


@pytest.mark.parametrize("block_rows", [0, 128])
@pytest.mark.parametrize("hadamard", [False, True])
def test_quantize_block_max_lands_in_top_binade_and_dequantizes_closely(block_rows, hadamard):
    x, _, _ = make_qkv_f32(2, 300, 3, 64, seed=11, outliers={"rate": 1e-3, "factor": 10})
    codes, desc = quantize(x, block_rows, hadamard, seed=5)
    vals = e4m3_decode(codes)
    # per tensor, amax / 448: the maximum maps to 448; per block, power-of-two
    # scales: the block maximum is in (224, 448] before rounding, [224, 448]
    # after it
    if block_rows == 0:
        assert desc.shape == (1,)
        assert np.abs(vals).max() == E4M3_MAX
    else:
        assert desc.shape == (2, 3, 3)
        for b in range(2):
            for h in range(3):
                for j in range(3):
                    blk = vals[b, j * 128:(j + 1) * 128, h]
                    assert E4M3_MAX / 2 <= np.abs(blk).max() <= E4M3_MAX
    ref = x.astype(np.float64)
    if hadamard:
        ref = ref @ hadamard_matrix(64, 5)
    dq = dequantize(codes, desc, block_rows)
    # every element within half an e4m3 step of its block's scale grid
    rel = np.abs(dq - ref)
    if block_rows == 0:
        bound = 2.0 ** -4 * np.abs(ref) + float(desc[0]) * 2.0 ** -10
    else:
        s = np.transpose(desc[:, :, np.arange(300) // 128], (0, 2, 1))[..., None]
        bound = 2.0 ** -4 * np.abs(ref) + s * 2.0 ** -10 + 1e-6 * s
    assert np.all(rel <= bound + 1e-12)


def test_quantize_exactly_representable_values_round_trip():
    vals = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448
    x = np.zeros((1, 128, 1, 128), np.float32)
    x[0, :, 0, :] = np.resize(vals, (128, 128)).astype(np.float32)
    codes, desc = quantize(x, 128)
    assert desc[0, 0, 0] == 1.0
    np.testing.assert_array_equal(e4m3_decode(codes), x.astype(np.float64))


def test_zero_block_uses_unit_scale():
    x = np.zeros((1, 130, 1, 64), np.float32)
    x[0, 128:, 0, :] = 3.0
    codes, desc = quantize(x, 128)
    assert desc[0, 0, 0] == 1.0 and np.all(codes[0, :128] == 0)
    assert desc[0, 0, 1] == np.float32(2.0 ** -7)  # 2^-8 < 3/448 <= 2^-7


def test_block_scale_is_the_smallest_power_of_two_covering_amax():
    from oracle.fp8 import block_scale
    for amax in (448.0, 449.0, 896.0, 1.0, 3.0, 7.0, 0.001, 1e5, 2.0 ** -100):
        s = float(block_scale(amax))
        m, _ = np.frexp(s)
        assert m == 0.5, (amax, s)                     # a power of two
        assert s >= amax / 448.0 and s / 2 < amax / 448.0, (amax, s)
    assert block_scale(448.0) == 1.0 and block_scale(448.5) == 2.0
    assert block_scale(0.0) == 1.0
    assert block_scale(1e-40) == np.float32(2.0 ** -126)   # clamped to the smallest normal


def test_emulated_fp8_attention_is_close_and_hadamard_helps_with_outliers():
    bits, (q, k, v) = make_qkv(1, 512, 2, 128, seed=0, outliers={"rate": 1e-3, "factor": 10})
    ref, lref = attention(q, k, v)
    rm = {}
    for name, br, had in (("tensor", 0, False), ("block+had", 128, True)):
        o, lse = emulated_fp8_attention(q, k, v, 1 / math.sqrt(128), False, br, had, 0)
        rm[name] = math.sqrt(np.mean((o - ref) ** 2))
    assert rm["block+had"] < 3e-2
    assert rm["block+had"] < rm["tensor"]
