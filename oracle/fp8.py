"""FP8 attention pieces of the oracle (test infrastructure only).

Sources:

* "FlashAttention-3 on Hopper", section 6.1: inputs use e4m3 (4 exponent
  bits, 3 mantissa bits, range +-448).
* Same page, section 6.3 (block quantization): one fp32 scale per B_M x d
  tile of Q and per B_N x d tile of K and V; the descales fold into the
  softmax scale (dQ * dK) and into the O rescale (dV).
* Same page, section 6.4, and "FlashAttention-3 paper review" (diycv.top),
  section "关键模块三：FP8 布局与误差控制": incoherent processing replaces
  Q <- Q M and K <- K M with M = (1/sqrt(d)) H D, H a +-1 Hadamard matrix and D
  a random +-1 diagonal; (QM)(KM)^T = Q K^T, so the scores are unchanged in
  exact arithmetic; x M costs O(d log d) with the fast Walsh-Hadamard
  transform. V is not transformed.
* "03 · FA3：Hopper 上的异步化与 overlap", section "4. FP8 的两个准确性问题与解法":
  Max_offset = 8 shifts the exponent of P so it uses the e4m3 range.

Readings of points the pages leave open:

* H is the Sylvester-ordered Hadamard matrix (H_1 = [1],
  H_2n = [[H_n, H_n], [H_n, -H_n]]), so d must be a power of two.
* M = H D / sqrt(d) exactly as the pages write it: a row vector x becomes
  ((x H) * sign) / sqrt(d).
* The diagonal signs come from SplitMix64 used as a counter-based generator:
  sign[i] = -1 if the top bit of splitmix64(seed + i) is set, else +1, where
  splitmix64(x) is the first output of a SplitMix64 generator whose state is x
  (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014).
* Scale rule: per 128-row block, scale = the smallest power of two >=
  amax(block) / 448 (the division in float32; at least 2^-126; 1 if
  amax = 0); per tensor, scale = amax / 448 (1 if amax = 0). Then code =
  e4m3_rne(saturate(x / scale)) and descale = scale. The pages fix a
  per-block scale but not its form. A power of two (an OCP MX E8M0 scale)
  divides exactly and can be applied by gfx950's scaled MFMA, so the
  attention kernel never rescales its accumulator when the V block changes;
  the block's largest value lands in (224, 448] instead of at 448. One
  scale per tensor never changes, so the per-tensor baseline keeps the
  plain amax / 448 (its accuracy is the pages' comparison point). Blocks are
  (b, h, 128 consecutive rows of N) over all d; "per tensor" means one scale
  for the whole tensor.
* The quantiser decides integer codes, so it computes in float32 (the
  kernel's precision) with the same operation order as the kernel: the FWHT
  butterflies in stages h = 1, 2, 4, ..., d/2 with (a + b, a - b), then one
  multiply by (+-1/sqrt(d)) rounded to float32, then an IEEE float32 division
  by the scale, then round-to-nearest-even to e4m3 with saturation at +-448.
"""
from __future__ import annotations

import numpy as np

from .attention import attention

__all__ = [
    "E4M3_MAX",
    "splitmix64",
    "hadamard_signs",
    "sylvester",
    "fwht",
    "e4m3_encode",
    "e4m3_decode",
    "quantize",
    "dequantize",
    "hadamard_matrix",
    "emulated_fp8_attention",
]

E4M3_MAX = 448.0
_MASK64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """First output of SplitMix64 with state ``x`` (Steele, Lea, Flood 2014)."""
    z = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def hadamard_signs(d: int, seed: int) -> np.ndarray:
    """The random +-1 diagonal D of M = H D / sqrt(d), as float64 (d,)."""
    return np.array([-1.0 if (splitmix64((seed + i) & _MASK64) >> 63) else 1.0 for i in range(d)])


def sylvester(d: int) -> np.ndarray:
    """Sylvester-ordered +-1 Hadamard matrix of order d (a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_matrix(d: int, seed: int) -> np.ndarray:
    """M = H D / sqrt(d) in float64 ("FlashAttention-3 on Hopper", section 6.4)."""
    return sylvester(d) * hadamard_signs(d, seed)[None, :] / np.sqrt(d)


def fwht(x: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis: returns x H.

    Butterfly stages h = 1, 2, ..., d/2; in each, the pair (a, b) = (x[i],
    x[i + h]) inside every block of 2h becomes (a + b, a - b). The arithmetic
    is done in ``dtype`` (float32 for the quantiser, float64 for checks).
    """
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 (e4m3fn) codes -> float64. S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3 codes, round to nearest even, saturating at +-448.

    Normal numbers have an unbiased exponent in [-6, 8] (bias 7) and 3
    fraction bits; below 2^-6 the grid is the subnormal step 2^-9. Every step
    here is exact in float64 except the final rounding, which is numpy's
    round-half-to-even.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # np.log2 can be off by one ulp near powers of two; fix the exponent exactly.
    e = np.where(np.exp2(e) > a, e - 1, e)
    e = np.where(np.exp2(e + 1) <= a, e + 1, e)
    e = np.maximum(e, -6.0)  # subnormal range shares the 2^-6 exponent
    step = np.exp2(e - 3.0)
    q = np.rint(a / step)  # integer multiple of the step, half to even
    # q in [8, 16] for normals (16 = carry into the next binade), [0, 8] for subnormals
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q)
    normal = q >= 8
    exp_field = np.where(normal, e + 7, 0).astype(np.int64)
    man_field = np.where(normal, q - 8, q).astype(np.int64)
    code = (exp_field << 3) | man_field
    code = np.where(code > 0x7E, 0x7E, code)  # saturate (0x7F would be NaN)
    code = code | np.where(sign, 0x80, 0)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def block_scale(amax):
    """The smallest power of two >= amax / 448 (float32 division), but at
    least 2^-126 (the smallest normal float32); 1 when amax is 0."""
    amax = np.float32(amax)
    if not amax > 0:
        return np.float32(1.0)
    r = np.float32(amax / np.float32(E4M3_MAX))
    m, e = np.frexp(r)  # r = m * 2^e with 0.5 <= m < 1
    p = r if m == 0.5 else np.float32(np.ldexp(np.float32(1.0), int(e)))
    return np.float32(max(p, np.float32(2.0 ** -126)))


def quantize(x, block_rows=128, hadamard=False, seed=0):
    """Block (or per-tensor) e4m3 quantisation of a (B, N, H, d) tensor.

    Returns (codes uint8 (B, N, H, d), descale float32). The descale array is
    (B, H, ceil(N / block_rows)) for block_rows > 0, or a (1,) array for the
    per-tensor case (block_rows = 0). Arithmetic is float32 in the order
    described in the module docstring.
    """
    x = np.asarray(x, dtype=np.float32)
    B, N, H, d = x.shape
    y = x
    if hadamard:
        y = fwht(x, np.float32)
        sign = hadamard_signs(d, seed).astype(np.float32)
        mult = (sign * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
        y = (y * mult).astype(np.float32)
    if block_rows == 0:
        amax = np.float32(np.max(np.abs(y))) if y.size else np.float32(0)
        scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
        codes = e4m3_encode((y / scale).astype(np.float32))
        return codes, np.array([scale], dtype=np.float32)
    nb = (N + block_rows - 1) // block_rows
    codes = np.zeros(x.shape, dtype=np.uint8)
    desc = np.zeros((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                blk = y[b, j * block_rows:(j + 1) * block_rows, h, :]
                amax = np.float32(np.max(np.abs(blk)))
                scale = block_scale(amax)
                codes[b, j * block_rows:(j + 1) * block_rows, h, :] = e4m3_encode((blk / scale).astype(np.float32))
                desc[b, h, j] = scale
    return codes, desc


def dequantize(codes, descale, block_rows=128):
    """Inverse of ``quantize`` up to rounding: codes * descale, float64."""
    vals = e4m3_decode(codes)
    if block_rows == 0:
        return vals * float(descale.reshape(-1)[0])
    B, N, H, d = codes.shape
    rows = np.arange(N) // block_rows
    scale = np.asarray(descale, dtype=np.float64)[:, :, rows]  # (B, H, N)
    return vals * np.transpose(scale, (0, 2, 1))[..., None]


def emulated_fp8_attention(q, k, v, alpha, causal=False, block_rows=128, hadamard=False, seed=0):
    """FP8-emulating reference (a debugging aid, not the graded oracle).

    Quantises Q and K (after the Hadamard transform when ``hadamard``) and V
    exactly as ``quantize`` does, dequantises, and runs the float64 attention
    definition. Since (QM)(KM)^T = Q K^T, its only departure from
    ``attention(q, k, v)`` is the quantisation error of the inputs; the
    GPU result additionally carries P's rounding to e4m3.
    """
    qc, qd = quantize(q, block_rows, hadamard, seed)
    kc, kd = quantize(k, block_rows, hadamard, seed)
    vc, vd = quantize(v, block_rows, False, seed)
    return attention(dequantize(qc, qd, block_rows), dequantize(kc, kd, block_rows),
                     dequantize(vc, vd, block_rows), alpha, causal)
