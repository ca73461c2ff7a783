"""Asymmetric per-(head, dim) INT8 quantisation with scale and offset tables (test infrastructure only).

Source: MindIE Turbo page "Attention量化" (attention quantization), tables 1 and 2:
the q, k and v activations carry a scale and an offset of shape
``[head_num, head_dim]``, stored as float16 (table 1) or bfloat16 (table 2).
The pages print the tables' shapes and dtypes but no formula and no way to
compute them; here they are inputs.

Readings:

* S1 the plain asymmetric INT8 code: ``code = clamp(rne(fl32(fl32(x / s) + o)),
  -128, 127)`` with ``s = scale[h, d]`` and ``o = offset[h, d]`` widened exactly
  to float32, ``x / s`` one correctly rounded float32 division, the addition one
  float32 addition and ``rne`` round half to even; a channel whose scale is 0
  gets code 0.
* S2 the value a code stands for is ``(code - o) * s``.
* S3 as for the symmetric K cache, only the first ``Dn`` features of a row are
  quantised; the last ``Dr`` (RoPE) are copied bit for bit.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .floats import bf16_bits_to_f32


def params_to_f32(bits, dtype: str) -> np.ndarray:
    """float32 value of a parameter table given as raw ``bfloat16`` or ``float16`` patterns."""
    b = np.asarray(bits).view(np.uint16) if np.asarray(bits).dtype == np.int16 else np.asarray(bits, dtype=np.uint16)
    if dtype == "bfloat16":
        return bf16_bits_to_f32(b)
    if dtype == "float16":
        return b.view(np.float16).astype(np.float32)
    raise ValueError("parameter tables are bfloat16 or float16")


def quantize_asym(k_bits, scale_bits, offset_bits, Dn: int, dtype: str = "bfloat16") -> Tuple[np.ndarray, np.ndarray]:
    """``(B,H,S,Dn+Dr)`` bf16 -> ``(codes (B,H,S,Dn) int8, rope (B,H,S,Dr) uint16)`` with ``[H, Dn]`` tables."""
    k_bits = np.asarray(k_bits).view(np.uint16) if np.asarray(k_bits).dtype == np.int16 else np.asarray(k_bits, dtype=np.uint16)
    B, H, S, _ = k_bits.shape
    s = params_to_f32(scale_bits, dtype).reshape(1, H, 1, Dn)
    o = params_to_f32(offset_bits, dtype).reshape(1, H, 1, Dn)
    x = bf16_bits_to_f32(k_bits[..., :Dn])
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = (x / s).astype(np.float32)                       # S1: float32 division
        z = (y + o).astype(np.float32)                       # S1: float32 addition
        code = np.clip(np.rint(z), -128.0, 127.0)            # S1: half to even, clamp
    code = np.where(s == np.float32(0.0), 0.0, code)
    return code.astype(np.int8), k_bits[..., Dn:].copy()


def dequantize_asym(codes, scale_bits, offset_bits, dtype: str = "bfloat16") -> np.ndarray:
    """float64 value of asymmetric codes ``(B,H,T,Dn)``: ``(code - o) * s`` (S2)."""
    codes = np.asarray(codes, dtype=np.int8)
    H, Dn = codes.shape[1], codes.shape[3]
    s = params_to_f32(scale_bits, dtype).astype(np.float64).reshape(1, H, 1, Dn)
    o = params_to_f32(offset_bits, dtype).astype(np.float64).reshape(1, H, 1, Dn)
    return (codes.astype(np.float64) - o) * s
