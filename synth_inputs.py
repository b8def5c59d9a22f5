"""Seeded synthetic inputs for attention tests and benchmarks.

This module only *generates* data: it draws Q, K, V, rounds them to the
16-bit storage format the kernels consume, and injects outliers. It holds
none of the attention method's arithmetic, so both the CPU oracle and the HIP
path can take their inputs from here without sharing any computation.

Recipe (the benchmark on the pages is a synthetic micro-benchmark: "FlashAttention-3
paper review", section on the experimental setup, and "FlashAttention-3 on
Hopper", section 6.4):

* ``rng = numpy.random.default_rng(seed)``; draw Q, then K, then V, each as
  ``rng.standard_normal((B, N, H, d), dtype=float32)`` (layout B, N, H, d).
* Round to bfloat16 (or float16) with round-to-nearest-even.
* The upstream gradient dO of the backward is drawn from its own generator,
  ``default_rng([seed, 1])``, as one ``standard_normal((B, N, H, d), float32)``
  draw rounded the same way, so it does not disturb the Q, K, V stream.
* Grouped heads / N_q != N_k (``make_qkv_gqa``): the same generator and
  order, with Q drawn as (B, N_q, H_q, d) and K, V as (B, N_k, H_kv, d).
* Packed variable-length batches (``make_seqlens``): per-sequence lengths
  i.i.d. uniform on [lo, hi] from ``default_rng([seed, 2])``; the packed
  tensors are ``make_qkv_gqa`` draws with B = 1 and N = the total length.
* Outliers (optional): an i.i.d. Bernoulli(rate) mask per element, independent
  for Q, K and V, drawn from the same generator after the base draws.
  ``kind="scale"`` multiplies the selected entries by ``factor`` (10);
  ``kind="additive"`` adds a N(0, factor**2) draw to them (the pages'
  N(0, 100) outlier model, read as variance 100).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "f32_to_f16_bits",
    "f16_bits_to_f32",
    "make_qkv",
    "make_qkv_f32",
    "make_dout",
    "make_qkv_gqa",
    "make_seqlens",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN stays NaN (quiet); infinities
    and values that round past the largest finite bfloat16 become infinities,
    which is what IEEE round-to-nearest-even gives.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    r = r.astype(np.uint32)
    r = np.where(nan, (u >> 16).astype(np.uint32) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast is RNE)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def make_qkv_f32(B, N, H, d, seed=0, outliers=None):
    """Draw float32 Q, K, V of shape (B, N, H, d) from ``default_rng(seed)``.

    ``outliers`` is None or a dict ``{"rate": 1e-3, "factor": 10.0,
    "kind": "scale" | "additive"}``.
    """
    rng = np.random.default_rng(seed)
    shape = (B, N, H, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if outliers:
        rate = float(outliers.get("rate", 1e-3))
        factor = float(outliers.get("factor", 10.0))
        kind = outliers.get("kind", "scale")
        out = []
        for t in (q, k, v):
            mask = rng.random(shape, dtype=np.float32) < rate
            if kind == "scale":
                t = np.where(mask, t * np.float32(factor), t)
            elif kind == "additive":
                extra = rng.standard_normal(shape, dtype=np.float32) * np.float32(factor)
                t = np.where(mask, t + extra, t)
            else:
                raise ValueError(f"unknown outlier kind {kind!r}")
            out.append(t.astype(np.float32))
        q, k, v = out
    return q, k, v


def make_qkv(B, N, H, d, seed=0, dtype="bf16", outliers=None):
    """Seeded Q, K, V rounded to a 16-bit storage type.

    Returns ``(bits, values)``: ``bits`` is a tuple of three uint16 arrays
    (the exact bytes handed to the GPU), ``values`` the same numbers widened
    to float64 (what the oracle consumes; the widening is exact).
    """
    q, k, v = make_qkv_f32(B, N, H, d, seed=seed, outliers=outliers)
    if dtype == "bf16":
        enc, dec = f32_to_bf16_bits, bf16_bits_to_f32
    elif dtype == "f16":
        enc, dec = f32_to_f16_bits, f16_bits_to_f32
    else:
        raise ValueError(dtype)
    bits = tuple(enc(t) for t in (q, k, v))
    vals = tuple(dec(b).astype(np.float64) for b in bits)
    return bits, vals


def make_dout(B, N, H, d, seed=0, dtype="bf16"):
    """Seeded upstream gradient dO, rounded like ``make_qkv``: (bits, values)."""
    rng = np.random.default_rng([seed, 1])
    g = rng.standard_normal((B, N, H, d), dtype=np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f16":
        bits = f32_to_f16_bits(g)
        return bits, f16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


def _round16(x, dtype):
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f16":
        bits = f32_to_f16_bits(x)
        return bits, f16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


def make_qkv_gqa(B, Nq, Nk, Hq, Hkv, d, seed=0, dtype="bf16"):
    """Q (B, Nq, Hq, d) and K, V (B, Nk, Hkv, d), drawn in that order from
    ``default_rng(seed)`` and rounded like ``make_qkv``: (bits, values)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Nq, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Nk, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, Nk, Hkv, d), dtype=np.float32)
    pairs = [_round16(t, dtype) for t in (q, k, v)]
    return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)


def make_seqlens(B, lo, hi, seed=0):
    """B sequence lengths, i.i.d. uniform integers on [lo, hi], and their
    prefix offsets (B + 1 int32 values starting at 0)."""
    rng = np.random.default_rng([seed, 2])
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return lens, cu
