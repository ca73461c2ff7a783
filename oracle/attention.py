"""Decode-phase attention over the quantised K cache, in float64 (test infrastructure only).

Sources: MindIE LLM page "FA3 quantization", overview paragraph (the INT8
K-nope / float K-rope cache exists to shrink KV-cache memory and speed up the
attention operator of the decode phase); MindIE page "Attention Quantization",
overview (same purpose for q/k/v).  The pages show no attention operator, so
this is the textbook single-query softmax attention over the dequantised cache.

Readings (also in the design doc):

* A1 the dequantised K-nope value is ``scale[h] * code`` (per head); the score
  is ``sm_scale * (q_nope . k_nope + q_rope . k_rope)``.
* A2 one query token per sequence attends to all ``T`` cached tokens (no mask).
* A3 Q, K-rope and V stay bf16; only K-nope is INT8 (the K-only variant).
* A4 the softmax scale is passed in; the workloads use ``1/sqrt(Dn + Dr)``.
"""
from __future__ import annotations

import numpy as np

from .floats import bf16_bits_to_f64
from .quant import dequantize_k_nope


def attention_fp64(q, k, v, sm_scale: float) -> np.ndarray:
    """Textbook softmax attention for one query per ``(b, h)``, all in float64.

    ``q (B,H,Dk)``, ``k (B,H,T,Dk)``, ``v (B,H,T,Dv)`` -> ``(B,H,Dv)``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scores = float(sm_scale) * np.einsum("bhd,bhtd->bht", q, k)
    scores = scores - scores.max(axis=-1, keepdims=True)
    weights = np.exp(scores)
    weights = weights / weights.sum(axis=-1, keepdims=True)
    return np.einsum("bht,bhtd->bhd", weights, v)


def decode_attn(q_bits, codes, scale, rope_bits, v_bits, sm_scale: float) -> np.ndarray:
    """Attention of bf16 ``q (B,H,Dn+Dr)`` over the INT8 K-nope + bf16 K-rope cache.

    ``codes (B,H,T,Dn) int8``, ``scale [H] float32``, ``rope_bits (B,H,T,Dr)`` and
    ``v_bits (B,H,T,Dv)`` bf16 patterns.  Returns float64 ``(B,H,Dv)``.
    """
    k_nope = dequantize_k_nope(codes, scale)
    k_rope = bf16_bits_to_f64(rope_bits)
    k = np.concatenate([k_nope, k_rope], axis=-1)
    return attention_fp64(bf16_bits_to_f64(q_bits), k, bf16_bits_to_f64(v_bits), float(np.float32(sm_scale)))
