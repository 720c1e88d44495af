"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the method (no frequencies, no rotation,
no softmax).  It only draws standard-normal values with numpy's PCG64 and
rounds them to the storage type the GPU consumes, so that both sides of a
parity check see bit-identical inputs:

* ``bf16`` inputs are drawn in fp32 and rounded to bfloat16 with
  round-to-nearest-even on the bit pattern; the fp32 view of the rounded
  value (exact) is what the oracle widens to fp64.
* ``f32`` inputs are used as drawn.

Seeds follow one convention everywhere: Q = seed_base + 0, K = +1, V = +2,
per-sequence ring heads = +3.
"""
from __future__ import annotations

import numpy as np

SEED_Q, SEED_K, SEED_V, SEED_RING = 0, 1, 2, 3


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round-to-nearest-even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to the fp32 values they encode (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal(shape, seed: int, dtype: str = "bf16"):
    """Draw N(0,1) values of ``shape``.

    Returns ``(values_f32, bits)``: ``values_f32`` are the exact values the GPU
    sees (as fp32), ``bits`` the uint16 bf16 patterns (``None`` for f32).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x, None
    if dtype != "bf16":
        raise ValueError(f"unsupported dtype {dtype!r}")
    bits = bf16_bits_from_f32(x)
    return f32_from_bf16_bits(bits), bits


def qkv(shape_q, shape_kv, dtype: str = "bf16", seed_base: int = 0):
    """Q, K, V draws with the fixed seed convention (seed_base + 0/1/2)."""
    q = normal(shape_q, seed_base + SEED_Q, dtype)
    k = normal(shape_kv, seed_base + SEED_K, dtype)
    v = normal(shape_kv, seed_base + SEED_V, dtype)
    return q, k, v


def ring_heads(batch: int, window: int, seed_base: int = 0) -> np.ndarray:
    """Per-sequence ring-buffer head of a sliding-window cache, uniform in [0, window)."""
    rng = np.random.default_rng(seed_base + SEED_RING)
    return rng.integers(0, window, size=batch, dtype=np.int64).astype(np.int32)


def sample_rows(n_rows: int, count: int, seed: int, must=()) -> np.ndarray:
    """A sorted, seeded sample of row indices in [0, n_rows) including ``must``."""
    rng = np.random.default_rng(seed)
    pick = set(int(r) for r in must if 0 <= r < n_rows)
    if count >= n_rows:
        return np.arange(n_rows)
    extra = rng.choice(n_rows, size=count, replace=False)
    pick.update(int(r) for r in extra)
    return np.array(sorted(pick), dtype=np.int64)


def e4m3_codes(shape, seed: int) -> np.ndarray:
    """Random 8-bit E4M3 codes (uint8) of moderate magnitude: random sign and
    mantissa, exponent field 4..9 (values between 2^-3 and about 7.5).  Only
    bit patterns are drawn; decoding them is the consumer's business."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    exp = rng.integers(4, 10, size=shape, dtype=np.uint8)
    man = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign << 7) | (exp << 3) | man


def e4m3_codes_banded(shape, seed: int, exp_fields) -> np.ndarray:
    """Random 8-bit E4M3 codes whose exponent field is fixed per leading
    index pair: exp_fields[b][h] (0..15) for codes [b, h, ...]; sign and
    mantissa random, the one NaN mantissa of field 15 excluded.  Only bit
    patterns are drawn."""
    rng = np.random.default_rng(seed)
    e = np.asarray(exp_fields, np.uint8).reshape(shape[:2] + (1,) * (len(shape) - 2))
    e = np.broadcast_to(e, shape)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    man = rng.integers(0, 8, size=shape, dtype=np.uint8)
    man = np.where(e == 15, man % 7, man).astype(np.uint8)
    return (sign << 7) | (e << 3) | man


def uniform_scales(shape, seed: int, lo: float = 0.05, hi: float = 0.5) -> np.ndarray:
    """fp32 values drawn uniformly from [lo, hi)."""
    return np.random.default_rng(seed).uniform(lo, hi, size=shape).astype(np.float32)
