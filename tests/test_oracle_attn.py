"""Pins for the oracle's float64 decode attention.

The pages show no attention operator (MindIE page "FA3 quantization" only says
the INT8 K cache serves decode-phase attention), so the oracle is the textbook
definition; it is pinned against torch's float64 scaled_dot_product_attention
on the CPU and against special cases with closed-form answers.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand_bits(rng, shape, std=1.0):
    return oracle.f32_to_bf16_bits_rne(rng.normal(size=shape).astype(np.float32) * np.float32(std))


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(31)
    B, H, T, Dk, Dv = 2, 3, 37, 24, 16
    q = rng.normal(size=(B, H, Dk)); k = rng.normal(size=(B, H, T, Dk)); v = rng.normal(size=(B, H, T, Dv))
    sm = 1 / math.sqrt(Dk)
    ours = oracle.attention_fp64(q, k, v, sm)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).unsqueeze(2), torch.from_numpy(k), torch.from_numpy(v), scale=sm
    ).squeeze(2).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(32)
    q = rng.normal(size=(1, 2, 8)); k = rng.normal(size=(1, 2, 1, 8)); v = rng.normal(size=(1, 2, 1, 5))
    np.testing.assert_allclose(oracle.attention_fp64(q, k, v, 0.3), v[:, :, 0], rtol=0, atol=1e-15)


def test_zero_query_is_mean_of_values():
    rng = np.random.default_rng(33)
    k = rng.normal(size=(1, 1, 50, 8)); v = rng.normal(size=(1, 1, 50, 4))
    out = oracle.attention_fp64(np.zeros((1, 1, 8)), k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_known_two_token_weights():
    # scores 0 and ln 3 -> weights 1/4 and 3/4
    q = np.array([[[1.0]]]); k = np.array([[[[0.0], [math.log(3.0)]]]])
    v = np.array([[[[4.0, 0.0], [0.0, 8.0]]]])
    out = oracle.attention_fp64(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], [1.0, 6.0], rtol=1e-14)


def test_dominant_token():
    rng = np.random.default_rng(34)
    k = rng.normal(size=(1, 1, 20, 4)) * 0.01
    k[0, 0, 13] = [50.0, 0, 0, 0]
    v = rng.normal(size=(1, 1, 20, 3))
    out = oracle.attention_fp64(np.array([[[1.0, 0, 0, 0]]]), k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0, 13], rtol=1e-15, atol=1e-15)


def test_decode_attn_is_attention_over_dequantised_cache():
    rng = np.random.default_rng(35)
    B, H, T, Dn, Dr, Dv = 2, 4, 64, 32, 16, 32
    qb = _rand_bits(rng, (B, H, Dn + Dr))
    codes = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    scale = np.exp(rng.uniform(-6, -2, size=H)).astype(np.float32)
    rope = _rand_bits(rng, (B, H, T, Dr))
    vb = _rand_bits(rng, (B, H, T, Dv))
    sm = np.float32(1 / math.sqrt(Dn + Dr))
    out = oracle.decode_attn(qb, codes, scale, rope, vb, sm)
    # independent assembly through torch fp64 SDPA on the dequantised K
    kd = torch.from_numpy(codes.astype(np.float64)) * torch.from_numpy(scale.astype(np.float64)).view(1, H, 1, 1)
    kr = torch.from_numpy(oracle.bf16_bits_to_f64(rope))
    k = torch.cat([kd, kr], dim=-1)
    q = torch.from_numpy(oracle.bf16_bits_to_f64(qb)).unsqueeze(2)
    v = torch.from_numpy(oracle.bf16_bits_to_f64(vb))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(sm)).squeeze(2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # factoring the per-head scale out of the nope dot product is the same attention
    qn = oracle.bf16_bits_to_f64(qb)[..., :Dn]
    s_factored = scale.astype(np.float64).reshape(1, H, 1) * np.einsum("bhd,bhtd->bht", qn, codes.astype(np.float64))
    s_elem = np.einsum("bhd,bhtd->bht", qn, kd.numpy())
    np.testing.assert_allclose(s_factored, s_elem, rtol=1e-13, atol=1e-13)


def test_bf16_helpers_roundtrip():
    x = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 1e-30, 65504.0], np.float32)
    bits = oracle.f32_to_bf16_bits_rne(x)
    back = oracle.bf16_bits_to_f32(bits)
    # values already representable in bf16 come back unchanged
    for a, b in zip(x[[0, 1, 2, 3, 4]], back[[0, 1, 2, 3, 4]]):
        assert a.view(np.uint32) == b.view(np.uint32)
    # rounding matches torch's float32 -> bfloat16 cast (round to nearest even)
    rng = np.random.default_rng(36)
    y = (rng.normal(size=10000) * np.exp(rng.uniform(-20, 20, size=10000))).astype(np.float32)
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits_rne(y), tb)


# ----------------------------------------------------------------------------- decode step


def _step_inputs(rng, B=3, H=4, T=40, Dn=32, Dr=16, Dv=32):
    k_full = _rand_bits(rng, (B, H, T, Dn + Dr), std=0.7)
    v_full = _rand_bits(rng, (B, H, T, Dv))
    qb = _rand_bits(rng, (B, H, Dn + Dr))
    scale = np.exp(rng.uniform(-6, -3, size=H)).astype(np.float32)
    return k_full, v_full, qb, scale


def test_append_at_last_position_reproduces_full_quantisation_and_attention():
    # The step writes the new token at position kv_len[b] = T-1: the cache must then equal
    # quantize_k of the whole K (a different call of the pinned quantiser, on the full
    # tensor), and the output the attention over all T tokens.
    rng = np.random.default_rng(41)
    B, H, T, Dn, Dr, Dv = 3, 4, 40, 32, 16, 32
    k_full, v_full, qb, scale = _step_inputs(rng, B, H, T, Dn, Dr, Dv)
    codes_full, rope_full = oracle.quantize_k(k_full, scale, Dn)
    # cache holding the first T-1 tokens and junk in the last slot
    codes = codes_full.copy()
    junk = rng.integers(-127, 128, size=(B, H, Dn)).astype(np.int8)
    codes[:, :, T - 1] = junk
    rope = rope_full.copy()
    rope[:, :, T - 1] = 0x7F00
    vb = v_full.copy()
    vb[:, :, T - 1] = 0x4000
    kv_len = np.full(B, T - 1, np.int32)
    out, c2, r2, v2 = oracle.decode_append_attn(qb, k_full[:, :, T - 1], v_full[:, :, T - 1], scale, codes, rope,
                                                vb, kv_len, np.float32(1 / math.sqrt(Dn + Dr)), Dn)
    np.testing.assert_array_equal(c2, codes_full)
    np.testing.assert_array_equal(r2, rope_full)
    np.testing.assert_array_equal(v2, v_full)
    ref = oracle.decode_attn(qb, codes_full, scale, rope_full, v_full, np.float32(1 / math.sqrt(Dn + Dr)))
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)
    # the input arrays are not modified
    np.testing.assert_array_equal(codes[:, :, T - 1], junk)
    assert (rope[:, :, T - 1] == 0x7F00).all() and (vb[:, :, T - 1] == 0x4000).all()


def test_append_to_empty_cache_returns_the_new_value():
    rng = np.random.default_rng(42)
    B, H, T, Dn, Dr, Dv = 2, 3, 8, 16, 8, 16
    k_full, v_full, qb, scale = _step_inputs(rng, B, H, T, Dn, Dr, Dv)
    codes = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    rope = _rand_bits(rng, (B, H, T, Dr))
    vb = _rand_bits(rng, (B, H, T, Dv))
    out, c2, _, _ = oracle.decode_append_attn(qb, k_full[:, :, 0], v_full[:, :, 0], scale, codes, rope, vb,
                                              np.zeros(B, np.int32), 0.3, Dn)
    # one token: its softmax weight is exactly 1
    np.testing.assert_array_equal(out, oracle.bf16_bits_to_f64(v_full[:, :, 0]))
    # rows other than position 0 are untouched
    np.testing.assert_array_equal(c2[:, :, 1:], codes[:, :, 1:])


def test_ragged_lengths_ignore_everything_past_the_length():
    rng = np.random.default_rng(43)
    B, H, T, Dn, Dr, Dv = 4, 2, 24, 16, 8, 16
    _, _, qb, scale = _step_inputs(rng, B, H, T, Dn, Dr, Dv)
    codes = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    rope = _rand_bits(rng, (B, H, T, Dr))
    vb = _rand_bits(rng, (B, H, T, Dv))
    kv_len = np.array([1, 7, 23, 24], np.int32)
    out, c2, r2, v2 = oracle.decode_append_attn(qb, None, None, scale, codes, rope, vb, kv_len, 0.25, Dn)
    # nothing is written without a new token
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(r2, rope)
    np.testing.assert_array_equal(v2, vb)
    # scrambling the capacity past each length changes nothing
    codes_x, rope_x, vb_x = codes.copy(), rope.copy(), vb.copy()
    for b, n in enumerate(kv_len):
        codes_x[b, :, n:] = 127
        rope_x[b, :, n:] = 0x4700  # 32768.0
        vb_x[b, :, n:] = 0xC700
    out_x, _, _, _ = oracle.decode_append_attn(qb, None, None, scale, codes_x, rope_x, vb_x, kv_len, 0.25, Dn)
    np.testing.assert_array_equal(out, out_x)
    # length 1: the first cached value
    np.testing.assert_array_equal(out[0], oracle.bf16_bits_to_f64(vb[0, :, 0]))
    # full length: the plain decode over the whole cache
    np.testing.assert_allclose(out[3], oracle.decode_attn(qb[3:], codes[3:], scale, rope[3:], vb[3:], 0.25)[0],
                               rtol=1e-14, atol=0)


def test_append_validates_lengths():
    rng = np.random.default_rng(44)
    B, H, T, Dn, Dr, Dv = 1, 1, 4, 16, 8, 16
    k_full, v_full, qb, scale = _step_inputs(rng, B, H, T, Dn, Dr, Dv)
    codes = np.zeros((B, H, T, Dn), np.int8)
    rope = np.zeros((B, H, T, Dr), np.uint16)
    vb = np.zeros((B, H, T, Dv), np.uint16)
    import pytest
    with pytest.raises(ValueError):
        oracle.decode_append_attn(qb, k_full[:, :, 0], v_full[:, :, 0], scale, codes, rope, vb,
                                  np.array([T], np.int32), 1.0, Dn)
    with pytest.raises(ValueError):
        oracle.decode_append_attn(qb, None, None, scale, codes, rope, vb, np.array([0], np.int32), 1.0, Dn)


# ----------------------------------------------------------------------------- paged cache


def _scatter_pages(cache, page_of, NP, P):
    """(B,H,T,D) contiguous cache -> (NP,H,P,D) pool with logical page j of sequence b at
    physical page page_of[b][j]; pages nobody owns hold a fixed junk pattern."""
    B, H, T, D = cache.shape
    pool = np.full((NP, H, P, D), 0x55 if cache.dtype == np.int8 else 0x7F7F, dtype=cache.dtype)
    for b in range(B):
        for j in range(T // P):
            for h in range(H):
                for r in range(P):
                    pool[page_of[b][j], h, r] = cache[b, h, j * P + r]
    return pool


def _paged_case(rng, B=3, H=2, P=16, MP=4, Dn=32, Dr=16, Dv=16, NP=None):
    T = MP * P
    NP = NP or B * MP + 3
    k_full, v_full, qb, scale = _step_inputs(rng, B, H, T, Dn, Dr, Dv)
    codes, rope = oracle.quantize_k(k_full, scale, Dn)
    page_of = rng.permutation(NP)[:B * MP].reshape(B, MP)
    return dict(k_full=k_full, v_full=v_full, qb=qb, scale=scale, codes=codes, rope=rope, page_of=page_of, T=T,
                pools=(_scatter_pages(codes, page_of, NP, P), _scatter_pages(rope, page_of, NP, P),
                       _scatter_pages(v_full, page_of, NP, P)))


def test_paged_step_equals_the_contiguous_step_on_scattered_pages():
    # the pools are built by a scatter written here, page by page and row by row; the paged
    # step must give the contiguous step's output, and its appended rows must land where the
    # scatter of the contiguous step's updated cache puts them
    rng = np.random.default_rng(51)
    B, H, P, MP, Dn, Dr, Dv = 3, 2, 16, 4, 32, 16, 16
    c = _paged_case(rng, B, H, P, MP, Dn, Dr, Dv)
    NP = c["pools"][0].shape[0]
    sm = np.float32(1 / math.sqrt(Dn + Dr))
    for kv_len, append in (([0, 17, 63], True), ([15, 16, 40], True), ([1, 33, 64], False)):
        kv_len = np.array(kv_len, np.int32)
        kn = c["k_full"][:, :, 5] if append else None
        vn = c["v_full"][:, :, 9] if append else None
        want, c2, r2, v2 = oracle.decode_append_attn(c["qb"], kn, vn, c["scale"], c["codes"], c["rope"],
                                                     c["v_full"], kv_len, sm, Dn)
        got, pc, pr, pv = oracle.decode_paged_attn(c["qb"], kn, vn, c["scale"], *c["pools"], c["page_of"], kv_len,
                                                   sm, Dn)
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)  # float64, summation order aside
        np.testing.assert_array_equal(pc, _scatter_pages(c2, c["page_of"], NP, P))
        np.testing.assert_array_equal(pr, _scatter_pages(r2, c["page_of"], NP, P))
        np.testing.assert_array_equal(pv, _scatter_pages(v2, c["page_of"], NP, P))


def test_paged_step_reads_only_the_pages_it_needs():
    rng = np.random.default_rng(52)
    B, H, P, MP, Dn, Dr, Dv = 2, 2, 16, 4, 16, 8, 16
    c = _paged_case(rng, B, H, P, MP, Dn, Dr, Dv)
    kv_len = np.array([20, 3], np.int32)  # pages 0-1 and page 0
    out, _, _, _ = oracle.decode_paged_attn(c["qb"], None, None, c["scale"], *c["pools"], c["page_of"], kv_len, 0.3, Dn)
    # table entries of pages past the length may be anything, even outside the pool
    bt = c["page_of"].copy()
    bt[0, 2:] = -7
    bt[1, 1:] = 10 ** 6
    out2, _, _, _ = oracle.decode_paged_attn(c["qb"], None, None, c["scale"], *c["pools"], bt, kv_len, 0.3, Dn)
    np.testing.assert_array_equal(out, out2)
    with pytest.raises(ValueError):
        oracle.decode_paged_attn(c["qb"], None, None, c["scale"], *c["pools"], bt, np.array([40, 3], np.int32), 0.3, Dn)


def test_paged_sequences_sharing_pages_agree():
    # two sequences whose block tables name the same pages read the same cache
    rng = np.random.default_rng(53)
    B, H, P, MP, Dn, Dr, Dv = 2, 3, 16, 3, 16, 8, 16
    c = _paged_case(rng, B, H, P, MP, Dn, Dr, Dv)
    bt = np.stack([c["page_of"][0], c["page_of"][0]])
    q = c["qb"].copy()
    q[1] = q[0]
    out, _, _, _ = oracle.decode_paged_attn(q, None, None, c["scale"], *c["pools"], bt, np.array([37, 37], np.int32),
                                            0.2, Dn)
    np.testing.assert_array_equal(out[0], out[1])


# ----------------------------------------------------------------------------- Q, K, V all INT8


def test_qkv8_attention_matches_sdpa_over_dequantised_tensors():
    rng = np.random.default_rng(45)
    B, H, T, Dn, Dr, Dv = 2, 3, 50, 32, 16, 32
    qc = rng.integers(-127, 128, size=(B, H, Dn)).astype(np.int8)
    qr = _rand_bits(rng, (B, H, Dr))
    kc = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    kr = _rand_bits(rng, (B, H, T, Dr))
    vc = rng.integers(-127, 128, size=(B, H, T, Dv)).astype(np.int8)
    sq, sk, sv = (np.exp(rng.uniform(-6, -2, size=H)).astype(np.float32) for _ in range(3))
    sm = np.float32(1 / math.sqrt(Dn + Dr))
    out = oracle.decode_attn_qkv8(qc, qr, sq, kc, sk, kr, vc, sv, sm)
    # independent assembly: torch float64 SDPA over tensors dequantised here
    s_ = lambda a: torch.from_numpy(a.astype(np.float64))
    q = torch.cat([s_(qc) * s_(sq).view(1, H, 1), torch.from_numpy(oracle.bf16_bits_to_f64(qr))], -1).unsqueeze(2)
    k = torch.cat([s_(kc) * s_(sk).view(1, H, 1, 1), torch.from_numpy(oracle.bf16_bits_to_f64(kr))], -1)
    v = s_(vc) * s_(sv).view(1, H, 1, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(sm)).squeeze(2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)
    # the integer form: q_nope . k_nope = sq*sk * sum(qc*kc), exact in integers
    ints = np.einsum("bhd,bhtd->bht", qc.astype(np.int64), kc.astype(np.int64))
    s_int = sq.astype(np.float64).reshape(1, H, 1) * sk.astype(np.float64).reshape(1, H, 1) * ints
    s_deq = np.einsum("bhd,bhtd->bht", q[..., 0, :Dn].numpy(), k[..., :Dn].numpy())
    np.testing.assert_allclose(s_int, s_deq, rtol=1e-13, atol=0)


def test_qkv8_with_unit_scales_is_plain_attention_over_codes():
    rng = np.random.default_rng(46)
    B, H, T, Dn, Dr, Dv = 1, 2, 9, 16, 8, 16
    qc = rng.integers(-3, 4, size=(B, H, Dn)).astype(np.int8)
    kc = rng.integers(-3, 4, size=(B, H, T, Dn)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(B, H, T, Dv)).astype(np.int8)
    zero_r = np.zeros((B, H, Dr), np.uint16)
    zero_kr = np.zeros((B, H, T, Dr), np.uint16)
    one = np.ones(H, np.float32)
    out = oracle.decode_attn_qkv8(qc, zero_r, one, kc, one, zero_kr, vc, one, 0.5)
    ref = oracle.attention_fp64(qc.astype(np.float64), kc.astype(np.float64), vc.astype(np.float64), 0.5)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=0)
    # and a single token returns its dequantised value exactly
    out1 = oracle.decode_attn_qkv8(qc, zero_r, one, kc[:, :, :1], one, zero_kr[:, :, :1], vc[:, :, :1],
                                   np.full(H, 0.25, np.float32), 0.5)
    np.testing.assert_array_equal(out1, 0.25 * vc[:, :, 0].astype(np.float64))


# ----------------------------------------------------------------------------- shared-latent (absorbed MLA) cache


def test_latent_decode_matches_sdpa_over_an_independently_assembled_cache():
    rng = np.random.default_rng(61)
    B, H, T, Dl, Dr = 2, 5, 40, 32, 16
    qb = _rand_bits(rng, (B, H, Dl + Dr))
    codes = rng.integers(-127, 128, size=(B, T, Dl)).astype(np.int8)
    rope = _rand_bits(rng, (B, T, Dr))
    s = np.float32(0.0173)
    sm = float(np.float32(1.0 / math.sqrt(192)))
    out = oracle.decode_attn_latent(qb, codes, s, rope, sm, Dl)
    q = torch.from_numpy(oracle.bf16_bits_to_f64(qb)).unsqueeze(2)                       # (B,H,1,D)
    lat = torch.from_numpy(codes.astype(np.float64)) * float(s)                          # (B,T,Dl)
    k = torch.cat([lat, torch.from_numpy(oracle.bf16_bits_to_f64(rope))], -1)           # (B,T,D)
    k = k.unsqueeze(1).expand(B, H, T, Dl + Dr)
    v = lat.unsqueeze(1).expand(B, H, T, Dl)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sm).squeeze(2).numpy()
    assert out.shape == (B, H, Dl)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-15)


def test_latent_decode_is_per_head_decode_of_the_latent_copied_to_every_head():
    # with a power-of-two scale the dequantised latent is exact in bf16, so the per-head
    # decode (K-nope codes + per-head scale, bf16 V) over the latent copied to every head
    # must give the same numbers
    rng = np.random.default_rng(62)
    B, H, T, Dl, Dr = 2, 4, 33, 16, 8
    qb = _rand_bits(rng, (B, H, Dl + Dr))
    codes = rng.integers(-127, 128, size=(B, T, Dl)).astype(np.int8)
    rope = _rand_bits(rng, (B, T, Dr))
    s = np.float32(2.0 ** -6)
    v_bits = oracle.f32_to_bf16_bits_rne(codes.astype(np.float32) * s)
    assert np.array_equal(oracle.bf16_bits_to_f64(v_bits), codes.astype(np.float64) * float(s))
    per_head = oracle.decode_attn(qb, np.repeat(codes[:, None], H, 1), np.full(H, s, np.float32),
                                  np.repeat(rope[:, None], H, 1), np.repeat(v_bits[:, None], H, 1), 0.3)
    np.testing.assert_allclose(oracle.decode_attn_latent(qb, codes, s, rope, 0.3, Dl), per_head, rtol=1e-13, atol=0)


def test_latent_decode_special_cases():
    rng = np.random.default_rng(63)
    B, H, T, Dl, Dr = 1, 3, 12, 16, 8
    codes = rng.integers(-127, 128, size=(B, T, Dl)).astype(np.int8)
    rope = _rand_bits(rng, (B, T, Dr))
    s = np.float32(0.05)
    # one token: every head returns its dequantised latent
    qb = _rand_bits(rng, (B, H, Dl + Dr))
    out1 = oracle.decode_attn_latent(qb, codes[:, :1], s, rope[:, :1], 0.2, Dl)
    np.testing.assert_array_equal(out1, np.broadcast_to(codes[:, None, 0].astype(np.float64) * float(s), (B, H, Dl)))
    # zero query: uniform weights, the mean of the dequantised latent
    q0 = np.zeros((B, H, Dl + Dr), np.uint16)
    out0 = oracle.decode_attn_latent(q0, codes, s, rope, 0.2, Dl)
    mean = codes.astype(np.float64).mean(axis=1) * float(s)
    np.testing.assert_allclose(out0, np.broadcast_to(mean[:, None], (B, H, Dl)), rtol=1e-13, atol=1e-16)
    # heads with equal query rows see the same weights
    qb[:, 2] = qb[:, 0]
    out = oracle.decode_attn_latent(qb, codes, s, rope, 0.2, Dl)
    np.testing.assert_array_equal(out[:, 2], out[:, 0])
    with pytest.raises(ValueError):
        oracle.decode_attn_latent(qb, codes[..., :8], s, rope, 0.2, Dl)
