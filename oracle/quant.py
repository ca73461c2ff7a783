"""INT8 quantisation of the non-RoPE part of K (test infrastructure only).

Sources: MindIE LLM page "FA3 quantization", overview paragraph (only the
non-RoPE slice of K is quantised to 8 bits, per head; the RoPE slice of K is
left unquantised); msModelSlim page "FA3量化", section 适用要求 (only symmetric
INT8) and section 算法流程 (``scale = abs_max / 127``).

The pages print no quantisation formula.  Readings:

* Q1 symmetric INT8 means no offset: ``code = clamp(round(x / scale), -127, 127)``;
  -128 is never produced and values beyond the calibrated range saturate.
* Q2 ``x / scale`` is one correctly rounded float32 division of the float32
  value of the bf16 input, and ``round`` is round-half-to-even applied to that
  float32 quotient.
* Q3 a head whose scale is 0 gets code 0 everywhere.
* Q4 the first ``Dn`` features of a K row are the non-RoPE part and the last
  ``Dr`` the RoPE part; the RoPE part is copied bit for bit, per head.

Fake quantisation (msModelSlim page "FA3量化", section 原理 -> 伪量化部署阶段: the
observer is replaced by a quantisation node built from the symmetric per-head
parameters).  The page gives no formula for the node; reading:

* F1 the node quantises as above and returns each code's value in the input's
  dtype: ``round_to_bf16(fl32(code * scale))``, one correctly rounded float32
  product, then round-half-to-even to bf16; the RoPE part passes unchanged.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .floats import bf16_bits_to_f32, bits16_to_f32, f32_to_bf16_bits_rne
from .layout import from_bhsd, to_bhsd


def quantize_k(k_bits, scale, Dn: int, dtype: str = "bf16", layout: str = "BHSD") -> Tuple[np.ndarray, np.ndarray]:
    """Split a 16-bit K tensor ``(B, H, S, Dn + Dr)`` into INT8 K-nope codes and K-rope.

    ``k_bits`` holds raw patterns of ``dtype`` ("bf16" or "f16"; Q2 takes their exact
    float32 value); ``scale`` is float32 ``[H]``.  Returns ``(codes (B,H,S,Dn) int8,
    rope (B,H,S,Dr) uint16 patterns)``, both in ``layout`` (for ``"BSHD"`` the input and
    outputs are ``(B, S, H, .)``, reading L4 of ``oracle.layout``).
    """
    k_bits = np.asarray(k_bits).view(np.uint16) if np.asarray(k_bits).dtype == np.int16 else np.asarray(k_bits, dtype=np.uint16)
    if k_bits.ndim != 4:
        raise ValueError("k must be (B, H, S, Dn + Dr)")
    if layout != "BHSD":
        codes, rope = quantize_k(to_bhsd(k_bits, layout), scale, Dn, dtype)
        return from_bhsd(codes, layout), from_bhsd(rope, layout)
    H = k_bits.shape[1]
    scale = np.asarray(scale, dtype=np.float32).reshape(H)
    x = bits16_to_f32(k_bits[..., :Dn], dtype)
    s = scale.reshape(1, H, 1, 1)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        quotient = (x / s).astype(np.float32)          # Q2: float32 division
        code = np.clip(np.rint(quotient), -127.0, 127.0)  # Q2: half-to-even, Q1: clamp
    code = np.where(s == np.float32(0.0), 0.0, code)       # Q3
    rope = k_bits[..., Dn:].copy()                          # Q4: bitwise copy
    return code.astype(np.int8), rope


def fake_quant(x_bits, scale, Dn: int) -> np.ndarray:
    """Quantise then dequantise the first ``Dn`` features of a bf16 ``(B, H, S, Dn + Dr)``
    tensor per head (F1); returns bf16 patterns of the same shape."""
    codes, rope = quantize_k(x_bits, scale, Dn)
    H = codes.shape[1]
    s = np.asarray(scale, dtype=np.float32).reshape(1, H, 1, 1)
    with np.errstate(over="ignore"):
        value = codes.astype(np.float32) * s                 # float32 product, correctly rounded
    return np.concatenate([f32_to_bf16_bits_rne(value), rope], axis=-1)


def dequantize_k_nope(codes, scale) -> np.ndarray:
    """float64 value represented by the INT8 K-nope cache: ``scale[h] * code``."""
    codes = np.asarray(codes, dtype=np.int8)
    H = codes.shape[1]
    s = np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(1, H, 1, 1)
    return s * codes.astype(np.float64)
