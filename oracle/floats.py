"""Bit-level float helpers for the oracle (test infrastructure only).

* bf16 is handled as raw ``uint16`` patterns; its exact float32 value is the
  pattern shifted into the high half of a 32-bit word.
* ``total_order_key`` maps float32 values to ``uint32`` keys whose unsigned
  order is the total order ``-inf < ... < -0.0 < +0.0 < ... < +inf`` used to
  sort a head's values (the pages say "sort" without naming an order for
  signed zeros; this reading makes -0.0 sort before +0.0).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact float32 value of bf16 patterns (uint16 or int16 array)."""
    b = np.asarray(bits).view(np.uint16) if np.asarray(bits).dtype == np.int16 else np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bf16 patterns."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def total_order_key(v) -> np.ndarray:
    """uint32 key increasing with the float32 total order (-0.0 below +0.0)."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    negative = (b >> np.uint32(31)) == np.uint32(1)
    return np.where(negative, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def key_to_f32(k) -> np.ndarray:
    """Inverse of :func:`total_order_key`."""
    k = np.asarray(k, dtype=np.uint32)
    from_negative = (k >> np.uint32(31)) == np.uint32(0)
    b = np.where(from_negative, ~k, k & np.uint32(0x7FFFFFFF)).astype(np.uint32)
    return b.view(np.float32)


def f16_bits_to_f32(bits) -> np.ndarray:
    """Exact float32 value of IEEE binary16 patterns, from the format's definition:
    sign s, 5-bit exponent e (bias 15), 10-bit fraction f; e = 0 is the subnormal range
    (-1)^s 2^-14 (f / 1024), e = 31 infinities and NaNs, otherwise (-1)^s 2^(e-15) (1 + f / 1024).
    Every binary16 value is exact in float32."""
    b = np.asarray(bits)
    b = b.view(np.uint16) if b.dtype == np.int16 else b.astype(np.uint16)
    s = (b >> np.uint16(15)).astype(np.int64)
    e = ((b >> np.uint16(10)) & np.uint16(0x1F)).astype(np.int64)
    f = (b & np.uint16(0x3FF)).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(f, -24), np.ldexp(1024.0 + f, (e - 25).astype(np.int32)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag).astype(np.float32)


def f16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of IEEE binary16 patterns."""
    return f16_bits_to_f32(bits).astype(np.float64)


def bits16_to_f32(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float32 value of 16-bit patterns of ``dtype`` ("bf16" or "f16")."""
    if dtype == "bf16":
        return bf16_bits_to_f32(bits)
    if dtype == "f16":
        return f16_bits_to_f32(bits)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def bits16_to_f64(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float64 value of 16-bit patterns of ``dtype`` ("bf16" or "f16")."""
    return bits16_to_f32(bits, dtype).astype(np.float64)
