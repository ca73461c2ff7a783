"""Decode-phase attention over the quantised K cache, in float64 (test infrastructure only).

Sources: MindIE LLM page "FA3 quantization", overview paragraph (the INT8
K-nope / float K-rope cache exists to shrink KV-cache memory and speed up the
attention operator of the decode phase); MindIE page "Attention Quantization",
overview (same purpose for q/k/v).  The pages show no attention operator, so
this is the textbook single-query softmax attention over the dequantised cache.

Readings:

* A1 the dequantised K-nope value is ``scale[h] * code`` (per head); the score
  is ``sm_scale * (q_nope . k_nope + q_rope . k_rope)``.
* A2 one query token per sequence attends to all ``T`` cached tokens (no mask).
* A3 Q, K-rope and V stay bf16; only K-nope is INT8 (the K-only variant).
* A4 the softmax scale is passed in; the workloads use ``1/sqrt(Dn + Dr)``.
"""
from __future__ import annotations

import numpy as np

from .floats import bf16_bits_to_f64, bits16_to_f64
from .layout import from_bhsd, to_bhsd
from .quant import dequantize_k_nope, quantize_k


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


def decode_attn(q_bits, codes, scale, rope_bits, v_bits, sm_scale: float, dtype: str = "bf16",
                layout: str = "BHSD") -> np.ndarray:
    """Attention of ``q (B,H,Dn+Dr)`` over the INT8 K-nope + 16-bit K-rope cache.

    ``codes (B,H,T,Dn) int8``, ``scale [H] float32``, ``rope_bits (B,H,T,Dr)`` and
    ``v_bits (B,H,T,Dv)``; q, K-rope and V are raw patterns of ``dtype`` ("bf16" or
    "f16").  With ``layout="BSHD"`` the three caches are ``(B,T,H,.)`` (reading L4 of
    ``oracle.layout``).  Returns float64 ``(B,H,Dv)``.
    """
    codes, rope_bits, v_bits = from_bhsd(codes, layout), from_bhsd(rope_bits, layout), from_bhsd(v_bits, layout)
    k_nope = dequantize_k_nope(codes, scale)
    k_rope = bits16_to_f64(rope_bits, dtype)
    k = np.concatenate([k_nope, k_rope], axis=-1)
    return attention_fp64(bits16_to_f64(q_bits, dtype), k, bits16_to_f64(v_bits, dtype), float(np.float32(sm_scale)))


def decode_append_attn(q_bits, k_new_bits, v_new_bits, scale, codes, rope_bits, v_bits, kv_len,
                       sm_scale: float, Dn: int, dtype: str = "bf16", layout: str = "BHSD"):
    """One decode step on a cache of capacity ``T`` with ragged lengths.

    Readings: A5 sequence ``b`` holds ``kv_len[b]`` cached
    tokens at positions ``0 .. kv_len[b]-1``; the rest of its capacity is not
    part of the attention.  A6 a new token (``k_new (B,H,Dn+Dr)``,
    ``v_new (B,H,Dv)`` bf16 patterns) goes to the next free position
    ``p = kv_len[b]``: its K-nope is quantised with the head's scale exactly as
    :func:`quantize_k` does, its K-rope and V are copied, and the step's query
    attends to positions ``0 .. p`` (the new token included).  Without a new
    token the query attends to ``0 .. kv_len[b]-1``.

    q, the new token and the cache's K-rope and V are raw patterns of ``dtype`` ("bf16" or
    "f16"); with ``layout="BSHD"`` the caches are ``(B,T,H,.)`` (reading L4 of
    ``oracle.layout``) and are returned in that layout.

    Returns ``(out (B,H,Dv) float64, codes, rope_bits, v_bits)`` with the
    cache arrays after the step (copies; the inputs are not modified).
    """
    if layout != "BHSD":
        out, c, r, v = decode_append_attn(q_bits, k_new_bits, v_new_bits, scale, to_bhsd(codes, layout),
                                          to_bhsd(rope_bits, layout), to_bhsd(v_bits, layout), kv_len, sm_scale, Dn,
                                          dtype)
        return out, from_bhsd(c, layout), from_bhsd(r, layout), from_bhsd(v, layout)
    codes = np.array(codes, dtype=np.int8, copy=True)
    rope_bits = np.array(rope_bits, dtype=np.uint16, copy=True)
    v_bits = np.array(v_bits, dtype=np.uint16, copy=True)
    B, H, T, _ = codes.shape
    Dv = v_bits.shape[-1]
    kv_len = np.asarray(kv_len, dtype=np.int64).reshape(B)
    out = np.zeros((B, H, Dv), dtype=np.float64)
    for b in range(B):
        p = int(kv_len[b])
        if k_new_bits is not None:
            if not 0 <= p < T:
                raise ValueError("appending needs 0 <= kv_len[b] < T")
            new_codes, new_rope = quantize_k(np.asarray(k_new_bits, dtype=np.uint16)[b][None, :, None, :], scale, Dn,
                                             dtype)
            codes[b, :, p, :] = new_codes[0, :, 0, :]
            rope_bits[b, :, p, :] = new_rope[0, :, 0, :]
            v_bits[b, :, p, :] = np.asarray(v_new_bits, dtype=np.uint16)[b]
            n = p + 1
        else:
            if not 1 <= p <= T:
                raise ValueError("attention needs 1 <= kv_len[b] <= T")
            n = p
        out[b] = decode_attn(np.asarray(q_bits)[b:b + 1], codes[b:b + 1, :, :n], scale, rope_bits[b:b + 1, :, :n],
                             v_bits[b:b + 1, :, :n], sm_scale, dtype)[0]
    return out, codes, rope_bits, v_bits


def decode_paged_attn(q_bits, k_new_bits, v_new_bits, scale, code_pool, rope_pool, v_pool, block_table, kv_len,
                      sm_scale: float, Dn: int):
    """:func:`decode_append_attn` over a paged cache.

    Reading P1: each cache is a pool of pages of ``P`` tokens laid
    out ``(num_pages, H, P, .)``; logical token ``t`` of sequence ``b`` is row ``t % P`` of
    physical page ``block_table[b, t // P]``.  The step reads the rows of tokens
    ``0 .. n-1`` (``n = kv_len[b] + 1`` with a new token, else ``kv_len[b]``), and the new
    token's rows are written at position ``kv_len[b]``.  Sequences are taken in order; an
    append into a page that another sequence reads is outside the reading (the steps of
    different sequences are independent).

    Returns ``(out (B,H,Dv) float64, code_pool, rope_pool, v_pool)`` after the step
    (copies; the inputs are not modified).
    """
    code_pool = np.array(code_pool, dtype=np.int8, copy=True)
    rope_pool = np.array(rope_pool, dtype=np.uint16, copy=True)
    v_pool = np.array(v_pool, dtype=np.uint16, copy=True)
    NP, H, P, _ = code_pool.shape
    block_table = np.asarray(block_table, dtype=np.int64)
    B, MP = block_table.shape
    T = MP * P
    kv_len = np.asarray(kv_len, dtype=np.int64).reshape(B)
    Dv = v_pool.shape[-1]
    out = np.zeros((B, H, Dv), dtype=np.float64)
    for b in range(B):
        p = int(kv_len[b])
        if k_new_bits is not None:
            if not 0 <= p < T:
                raise ValueError("appending needs 0 <= kv_len[b] < T")
            n = p + 1
        else:
            if not 1 <= p <= T:
                raise ValueError("attention needs 1 <= kv_len[b] <= T")
            n = p
        pages = block_table[b, :(n + P - 1) // P]
        if np.any(pages < 0) or np.any(pages >= NP):
            raise ValueError("block table entry outside the pool")
        if k_new_bits is not None:
            new_codes, new_rope = quantize_k(np.asarray(k_new_bits, dtype=np.uint16)[b][None, :, None, :], scale, Dn)
            pg, row = block_table[b, p // P], p % P
            code_pool[pg, :, row, :] = new_codes[0, :, 0, :]
            rope_pool[pg, :, row, :] = new_rope[0, :, 0, :]
            v_pool[pg, :, row, :] = np.asarray(v_new_bits, dtype=np.uint16)[b]
        # the sequence's first n tokens, in logical order: (H, n, .)
        t = np.arange(n)
        pg, row = block_table[b, t // P], t % P
        codes = code_pool[pg, :, row, :].transpose(1, 0, 2)
        rope = rope_pool[pg, :, row, :].transpose(1, 0, 2)
        vals = v_pool[pg, :, row, :].transpose(1, 0, 2)
        out[b] = decode_attn(np.asarray(q_bits)[b:b + 1], codes[None], scale, rope[None], vals[None], sm_scale)[0]
    return out, code_pool, rope_pool, v_pool


def decode_attn_qkv8(q_codes, q_rope_bits, scale_q, k_codes, scale_k, k_rope_bits, v_codes, scale_v,
                     sm_scale: float) -> np.ndarray:
    """Attention with Q, K and V all per-head INT8 (the RoPE parts of Q and K in bf16).

    Readings: A8 Q's non-RoPE part and all of V are quantised
    per head with the same symmetric formula as K (``quantize_k``); their
    dequantised values are ``scale_q[h] * code`` and ``scale_v[h] * code``; the
    RoPE parts of Q and K stay bf16.  The attention is the textbook one over the
    dequantised tensors, in float64.

    ``q_codes (B,H,Dn) int8``, ``q_rope_bits (B,H,Dr)``, ``k_codes (B,H,T,Dn) int8``,
    ``k_rope_bits (B,H,T,Dr)``, ``v_codes (B,H,T,Dv) int8``; scales float32 ``[H]``.
    Returns float64 ``(B,H,Dv)``.
    """
    q_codes = np.asarray(q_codes, dtype=np.int8)
    B, H, Dn = q_codes.shape
    q_nope = dequantize_k_nope(q_codes.reshape(B, H, 1, Dn), scale_q).reshape(B, H, Dn)
    q = np.concatenate([q_nope, bf16_bits_to_f64(q_rope_bits)], axis=-1)
    k = np.concatenate([dequantize_k_nope(k_codes, scale_k), bf16_bits_to_f64(k_rope_bits)], axis=-1)
    v = dequantize_k_nope(v_codes, scale_v)
    return attention_fp64(q, k, v, float(np.float32(sm_scale)))


def decode_attn_asym(q_bits, codes, scale_bits, offset_bits, rope_bits, v_bits, sm_scale: float,
                     dtype: str = "bfloat16") -> np.ndarray:
    """Attention of bf16 ``q (B,H,Dn+Dr)`` over an asymmetric per-(head, dim) INT8 K-nope cache.

    Same as :func:`decode_attn` with the K-nope value ``(code - offset[h,d]) * scale[h,d]``
    (readings S1-S2 of ``oracle.asym``); K-rope and V bf16.  Returns float64 ``(B,H,Dv)``.
    """
    from .asym import dequantize_asym
    k = np.concatenate([dequantize_asym(codes, scale_bits, offset_bits, dtype), bf16_bits_to_f64(rope_bits)], axis=-1)
    return attention_fp64(bf16_bits_to_f64(q_bits), k, bf16_bits_to_f64(v_bits), float(np.float32(sm_scale)))


def decode_attn_latent(q_bits, codes, scale, rope_bits, sm_scale: float, Dl: int) -> np.ndarray:
    """Decode over a shared-latent (absorbed MLA) cache: every head of a sequence reads the same rows.

    MindIE LLM page "FA3 quantization", overview (MLA attention; only the non-RoPE part of
    K goes to INT8, the RoPE part stays floating point).  The pages give no layout for the
    shared latent; the readings are:

    * L1 the latent rows ``[c | k_rope]`` of a sequence form one head shared by all query
      heads, so the per-head method runs with one head: ``c`` holds INT8 codes with one
      scale ``s`` (from the same calibration and quantiser), ``k_rope`` stays bf16;
    * L2 the query is already absorbed: ``q (B,H,Dl+Dr)`` bf16 is ``[q_abs | q_rope]``; the
      score of token t is ``sm * (s * <q_abs, c_t> + <q_rope, r_t>)`` and the value is the
      dequantised latent ``s * c_t``;
    * L3 the output is the latent-space attention ``(B,H,Dl)``, float64 here (the
      up-projection to the head's value space is outside the path).

    ``codes (B,T,Dl)`` int8, ``rope_bits (B,T,Dr)`` bf16 patterns, ``scale`` a scalar.
    """
    q = bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16))
    codes = np.asarray(codes, dtype=np.int8)
    B, H, _ = q.shape
    T = codes.shape[1]
    if codes.shape != (B, T, Dl):
        raise ValueError("codes must be (B, T, Dl)")
    s = float(np.float32(scale))
    c = codes.astype(np.float64) * s                                   # L1: dequantised latent
    r = bf16_bits_to_f64(np.asarray(rope_bits, dtype=np.uint16)).reshape(B, T, -1)
    k = np.concatenate([c, r], axis=-1)                                # (B,T,Dl+Dr), one K for every head
    # textbook softmax attention with that K and V = c (L2) shared by all heads of a sequence
    scores = float(np.float32(sm_scale)) * np.einsum("bhd,btd->bht", q, k)   # sm as the float32 callers pass
    scores = scores - scores.max(axis=-1, keepdims=True)
    weights = np.exp(scores)
    weights = weights / weights.sum(axis=-1, keepdims=True)
    return np.einsum("bht,btd->bhd", weights, c)
