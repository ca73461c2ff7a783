"""Pins for the oracle's K quantisation.

Sources: MindIE LLM page "FA3 quantization" (overview: non-RoPE K to 8 bits per
head, RoPE K untouched); msModelSlim page "FA3量化" (适用要求: INT8 symmetric
only; 算法流程: scale = abs_max/127).  The code of each element is checked
against an independent exact-rational computation of the float32 quotient and
Python's half-to-even ``round``.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bits16(x_f32):
    """bf16 patterns of float32 values that are exactly representable in bf16."""
    u = np.asarray(x_f32, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _round_f32(q: Fraction) -> float:
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.asarray(v, np.float32).view(np.uint32)) & 1))
    return float(best)


def _code(x: float, s: float) -> int:
    if s == 0.0:
        return 0
    qf = _round_f32(Fraction(x) / Fraction(s))
    r = round(qf)  # Python rounds half to even
    return max(-127, min(127, r))


def _random_k(rng, B, H, S, Dn, Dr, sigma):
    x = rng.normal(size=(B, H, S, Dn + Dr)).astype(np.float32) * sigma.reshape(1, H, 1, 1)
    return oracle.f32_to_bf16_bits_rne(x).reshape(B, H, S, Dn + Dr)


def test_codes_match_exact_rational_rounding():
    rng = np.random.default_rng(21)
    B, H, S, Dn, Dr = 1, 3, 40, 16, 8
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    scale = (sigma * np.float32(3.0) / np.float32(127)).astype(np.float32)
    codes, rope = oracle.quantize_k(k, scale, Dn)
    xs = oracle.bf16_bits_to_f32(k[..., :Dn])
    for idx in np.ndindex(codes.shape):
        assert codes[idx] == _code(float(xs[idx]), float(scale[idx[1]])), idx


def test_half_integer_quotients_round_to_even():
    # x = (n + 1/2) * s exactly: 0.5->0, 1.5->2, 2.5->2, -2.5->-2, 126.5->126, 127.5 -> clamp 127
    s = np.float32(0.25)
    vals = np.array([0.5, 1.5, 2.5, -2.5, 3.5, -0.5, 126.5, 127.5, -127.5, 1000.0], np.float32) * s
    k = _bits16(vals).reshape(1, 1, 1, -1)
    k = np.concatenate([k, np.zeros((1, 1, 1, 8), np.uint16)], axis=-1)
    codes, _ = oracle.quantize_k(k, np.array([s]), vals.size)
    assert codes.reshape(-1).tolist() == [0, 2, 2, -2, 4, 0, 126, 127, -127, 127]


def test_symmetric_range_saturation_and_error_bound():
    rng = np.random.default_rng(22)
    B, H, S, Dn, Dr = 2, 4, 64, 32, 16
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    # plant outliers at +-40 sigma (bf16-rounded) in the nope part
    x = oracle.bf16_bits_to_f32(k).copy()
    x[0, :, 3, 5] = 40 * sigma
    x[1, :, 7, 9] = -40 * sigma
    k = oracle.f32_to_bf16_bits_rne(x)
    absmax = (4 * sigma).astype(np.float32)
    scale = oracle.qparams(-absmax, absmax)
    codes, rope = oracle.quantize_k(k, scale, Dn)
    assert codes.dtype == np.int8
    assert codes.min() >= -127 and codes.max() <= 127  # -128 never produced
    assert np.all(codes[0, :, 3, 5] == 127) and np.all(codes[1, :, 7, 9] == -127)
    xn = oracle.bf16_bits_to_f32(k[..., :Dn]).astype(np.float64)
    s64 = scale.astype(np.float64).reshape(1, H, 1, 1)
    inside = np.abs(xn) <= 127 * s64
    err = np.abs(xn - codes.astype(np.float64) * s64)
    assert np.all(err[inside] <= (s64 * (0.5 + 2.0 ** -17) * np.ones_like(xn))[inside])
    # the RoPE slice is a byte-for-byte copy
    assert rope.dtype == np.uint16
    assert rope.tobytes() == np.ascontiguousarray(k[..., Dn:]).tobytes()


def test_zero_scale_head_gives_zero_codes():
    rng = np.random.default_rng(23)
    k = _random_k(rng, 1, 2, 8, 16, 8, np.ones(2, np.float32))
    codes, _ = oracle.quantize_k(k, np.array([0.0, 1.0], np.float32), 16)
    assert np.all(codes[:, 0] == 0)
    assert np.any(codes[:, 1] != 0)


def test_quantize_roundtrip_with_calibrated_scale():
    # scale from the oracle's own calibration of the same data: every value inside
    # the recall window maps inside [-127, 127] without saturation error.
    rng = np.random.default_rng(24)
    B, H, S, Dn, Dr = 1, 4, 64, 32, 16
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    xn = oracle.bf16_bits_to_f32(k[..., :Dn])
    lo, hi = oracle.calibrate(xn, 0.99)
    scale = oracle.qparams(lo, hi)
    codes, _ = oracle.quantize_k(k, scale, Dn)
    for h in range(H):
        sel = (xn[:, h] >= lo[h]) & (xn[:, h] <= hi[h])
        err = np.abs(xn[:, h][sel].astype(np.float64) - codes[:, h][sel] * float(scale[h]))
        assert err.max() <= float(scale[h]) * (0.5 + 2.0 ** -17)


@pytest.mark.parametrize("bad", [np.zeros((2, 3, 4)), np.zeros((1, 2, 3, 4, 5))])
def test_shape_validation(bad):
    with pytest.raises(ValueError):
        oracle.quantize_k(bad.astype(np.uint16), np.ones(3, np.float32), 2)


# ----------------------------------------------------------------------------- asymmetric per-(head, dim)
# MindIE Turbo page "Attention量化", tables 1 and 2: scale and offset tables [heads, head_dim] in
# float16 or bfloat16.  The quantiser is checked against exact rational arithmetic (float32
# division, then float32 addition, then half-to-even), closed forms and the symmetric quantiser.


def _f32(q: Fraction) -> Fraction:
    return Fraction(_round_f32(q))


def _code_asym(x: float, s: float, o: float) -> int:
    if s == 0.0:
        return 0
    y = _f32(Fraction(x) / Fraction(s))
    z = _f32(y + Fraction(o))
    return max(-128, min(127, round(z)))


def _bf16_params(rng, H, Dn, lo, hi):
    return oracle.f32_to_bf16_bits_rne(rng.uniform(lo, hi, size=(H, Dn)).astype(np.float32))


def test_asym_codes_match_exact_rational_arithmetic():
    rng = np.random.default_rng(51)
    B, H, S, Dn, Dr = 2, 3, 20, 16, 8
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    scale = _bf16_params(rng, H, Dn, 0.005, 0.05)
    offset = _bf16_params(rng, H, Dn, -20.0, 20.0)
    codes, rope = oracle.quantize_asym(k, scale, offset, Dn)
    xs = oracle.bf16_bits_to_f32(k[..., :Dn])
    sf, of = oracle.bf16_bits_to_f32(scale), oracle.bf16_bits_to_f32(offset)
    for idx in np.ndindex(codes.shape):
        b, h, s_, d = idx
        assert codes[idx] == _code_asym(float(xs[idx]), float(sf[h, d]), float(of[h, d])), idx
    np.testing.assert_array_equal(rope, k[..., Dn:])


def test_asym_hand_values_and_saturation():
    # s = 1, o = 0.5: z = x + 0.5 -> 0.5 + 0.5 = 1, -1.0 + 0.5 = -0.5 -> -0 (half to even), 2.0 + 0.5 = 2.5 -> 2
    # -129 + 0.5 = -128.5 rounds half to even to -128 (inside the range); -1000 saturates
    x = np.array([0.5, -1.0, 2.0, 1000.0, -1000.0, 126.5, -129.0], np.float32)
    k = _bits16(x).reshape(1, 1, 1, -1)
    Dn = x.size
    one = _bits16(np.ones((1, Dn), np.float32))
    half = _bits16(np.full((1, Dn), 0.5, np.float32))
    codes, _ = oracle.quantize_asym(k, one, half, Dn)
    assert codes.reshape(-1).tolist() == [1, 0, 2, 127, -128, 127, -128]
    # a channel whose scale is 0 gets code 0 whatever its input and offset
    zero_first = one.copy()
    zero_first[0, 0] = 0
    codes, _ = oracle.quantize_asym(k, zero_first, half, Dn)
    assert codes.reshape(-1).tolist() == [0, 0, 2, 127, -128, 127, -128]


def test_asym_without_offset_is_the_symmetric_quantiser_inside_its_range():
    # offset 0 and a per-head scale copied to every dim: the same codes as quantize_k wherever
    # |x / s| rounds inside +-127 (the symmetric range); only the asymmetric -128 differs
    rng = np.random.default_rng(52)
    B, H, S, Dn, Dr = 2, 4, 30, 32, 16
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    s_head = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits_rne((sigma * np.float32(3.0) / np.float32(127))))
    sym, _ = oracle.quantize_k(k, s_head, Dn)
    scale_tab = np.repeat(oracle.f32_to_bf16_bits_rne(s_head).reshape(H, 1), Dn, axis=1)
    asym, _ = oracle.quantize_asym(k, scale_tab, np.zeros((H, Dn), np.uint16), Dn)
    inside = np.abs(asym.astype(np.int32)) <= 127
    np.testing.assert_array_equal(asym[inside], sym[inside])
    assert np.all(sym[~inside] == -127) and np.all(asym[~inside] == -128)


def test_asym_roundtrip_error_bound_and_float16_tables():
    rng = np.random.default_rng(53)
    B, H, S, Dn, Dr = 1, 2, 64, 16, 0
    x = rng.uniform(-3, 5, size=(B, H, S, Dn)).astype(np.float32)
    k = oracle.f32_to_bf16_bits_rne(x).reshape(B, H, S, Dn)
    xf = oracle.bf16_bits_to_f32(k).astype(np.float64)
    lo, hi = -3.0, 5.0
    s = np.float32((hi - lo) / 255.0)
    o = np.float32(-128.0 - np.rint(lo / s))
    for dtype, conv in (("float16", lambda a: np.asarray(a, np.float16).view(np.uint16)),
                        ("bfloat16", lambda a: oracle.f32_to_bf16_bits_rne(np.asarray(a, np.float32)))):
        sb = conv(np.full((H, Dn), s, np.float32))
        ob = conv(np.full((H, Dn), o, np.float32))
        codes, _ = oracle.quantize_asym(k, sb, ob, Dn, dtype)
        deq = oracle.dequantize_asym(codes, sb, ob, dtype)
        s_used = float(oracle.params_to_f32(sb, dtype)[0, 0])
        # every value inside the representable range comes back within half a step (plus
        # the float32 rounding of the quotient and of the addition)
        assert np.max(np.abs(deq - xf)) <= s_used * (0.5 + 1e-3)
    # float16 patterns are read as float16 values
    np.testing.assert_array_equal(oracle.params_to_f32(np.array([0x3C00, 0xC000], np.uint16), "float16"),
                                  np.array([1.0, -2.0], np.float32))


def test_asym_decode_is_attention_over_dequantised_cache():
    import math
    import torch
    rng = np.random.default_rng(54)
    B, H, T, Dn, Dr, Dv = 2, 3, 40, 32, 16, 32
    q = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, H, Dn + Dr)).astype(np.float32))
    codes = rng.integers(-128, 128, size=(B, H, T, Dn)).astype(np.int8)
    scale = _bf16_params(rng, H, Dn, 0.001, 0.02)
    offset = _bf16_params(rng, H, Dn, -30.0, 30.0)
    rope = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, H, T, Dr)).astype(np.float32))
    v = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, H, T, Dv)).astype(np.float32))
    sm = np.float32(1 / math.sqrt(Dn + Dr))
    out = oracle.decode_attn_asym(q, codes, scale, offset, rope, v, sm)
    sf = torch.from_numpy(oracle.bf16_bits_to_f32(scale).astype(np.float64)).view(1, H, 1, Dn)
    of = torch.from_numpy(oracle.bf16_bits_to_f32(offset).astype(np.float64)).view(1, H, 1, Dn)
    kd = (torch.from_numpy(codes.astype(np.float64)) - of) * sf
    k = torch.cat([kd, torch.from_numpy(oracle.bf16_bits_to_f64(rope))], -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(oracle.bf16_bits_to_f64(q)).unsqueeze(2), k, torch.from_numpy(oracle.bf16_bits_to_f64(v)),
        scale=float(sm)).squeeze(2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # zero offsets and one scale per head: the symmetric decode
    s_head = oracle.bf16_bits_to_f32(scale)[:, 0]
    tab = np.repeat(scale[:, :1], Dn, axis=1)
    np.testing.assert_allclose(oracle.decode_attn_asym(q, codes, tab, np.zeros((H, Dn), np.uint16), rope, v, sm),
                               oracle.decode_attn(q, codes, s_head, rope, v, sm), rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------- fake quantisation
# msModelSlim page "FA3量化", 原理 -> 伪量化部署阶段: the observer becomes a quantisation node
# built from the symmetric per-head parameters; reading F1: each code's value scale * code,
# one float32 product, rounded to bf16.  Checked against exact rationals rounded by hand,
# hand values, and the invariants any quantise-dequantise pair must keep.


def _round_sig(q: Fraction, p: int) -> Fraction:
    """q rounded to p significant bits, ties to even (normal range, no overflow)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - p + 1)
    n, rem = divmod(a, unit)
    n = int(n)
    if rem > unit / 2 or (rem == unit / 2 and n % 2 == 1):
        n += 1
    return sign * n * unit


def _fake_value(x: float, s: float) -> float:
    c = _code(x, s)
    return float(_round_sig(_round_sig(Fraction(c) * Fraction(s), 24), 8))


def test_fake_quant_hand_values():
    # scale 0.25: quotients 2, 4, -11, 400 (-> 127), 1.5 (-> 2), 2.5 (-> 2), -1.5 (-> -2), -127.5 (-> -127)
    x = np.array([0.5, 1.0, -2.75, 100.0, 0.375, 0.625, -0.375, -31.875] * 2, np.float32)
    k = _bits16(x).reshape(1, 1, 1, 16)
    got = oracle.bf16_bits_to_f32(oracle.fake_quant(k, np.array([0.25], np.float32), 16)).reshape(-1)
    want = np.array([0.5, 1.0, -2.75, 31.75, 0.5, 0.5, -0.5, -31.75] * 2, np.float32)
    np.testing.assert_array_equal(got, want)
    # scale fl32(0.01): 5.0 saturates to 127 * s = 1.26999997..., whose nearest bf16 is 1.2734375
    y = oracle.bf16_bits_to_f32(oracle.fake_quant(_bits16(np.full(16, 5.0, np.float32)).reshape(1, 1, 1, 16),
                                                  np.array([0.01], np.float32), 16))
    assert np.all(y == np.float32(1.2734375))


def test_fake_quant_matches_exact_double_rounding():
    rng = np.random.default_rng(31)
    B, H, S, Dn, Dr = 1, 4, 24, 16, 8
    sigma = np.exp(rng.uniform(-3, 3, size=H)).astype(np.float32)
    k = _random_k(rng, B, H, S, Dn, Dr, sigma)
    scale = (sigma * np.exp(rng.uniform(0.0, 2.0, size=H)) / 127).astype(np.float32)  # arbitrary float32 scales
    y = oracle.fake_quant(k, scale, Dn)
    assert y.shape == k.shape and y.dtype == np.uint16
    ys = oracle.bf16_bits_to_f32(y[..., :Dn])
    xs = oracle.bf16_bits_to_f32(k[..., :Dn])
    for idx in np.ndindex(ys.shape):
        assert ys[idx] == _fake_value(float(xs[idx]), float(scale[idx[1]])), idx
    np.testing.assert_array_equal(y[..., Dn:], k[..., Dn:])


def test_fake_quant_is_idempotent_and_monotone():
    # bf16 rounding moves scale * code by at most half an ulp, 2^-8 of itself: under
    # 127 * 2^-8 < 0.4961 scale for |code| <= 127 (plus float32 rounding far below the
    # remaining margin), so quantising a fake-quantised value returns the same code and value
    rng = np.random.default_rng(32)
    H, S, Dn = 6, 200, 32
    sigma = np.exp(rng.uniform(-4, 4, size=H)).astype(np.float32)
    k = _random_k(rng, 1, H, S, Dn, 0, sigma)
    scale = (sigma * np.exp(rng.uniform(-1.0, 2.0, size=H)) / 127).astype(np.float32)
    y = oracle.fake_quant(k, scale, Dn)
    np.testing.assert_array_equal(oracle.fake_quant(y, scale, Dn), y)
    xs = oracle.bf16_bits_to_f32(k).astype(np.float64)
    ys = oracle.bf16_bits_to_f32(y).astype(np.float64)
    for h in range(H):
        order = np.argsort(xs[0, h].reshape(-1), kind="stable")
        assert np.all(np.diff(ys[0, h].reshape(-1)[order]) >= 0), h


def test_fake_quant_error_bound_saturation_zero_scale():
    rng = np.random.default_rng(33)
    H, S, Dn, Dr = 4, 256, 16, 8
    sigma = np.ones(H, np.float32)
    k = _random_k(rng, 1, H, S, Dn, Dr, sigma)
    scale = np.array([0.02, 0.005, 0.0, 1.0 / 127], np.float32)  # head 2 has an empty range
    y = oracle.fake_quant(k, scale, Dn)
    xs = oracle.bf16_bits_to_f32(k[..., :Dn]).astype(np.float64)
    ys = oracle.bf16_bits_to_f32(y[..., :Dn]).astype(np.float64)
    for h in (0, 1, 3):
        s = float(scale[h])
        x, v = xs[0, h], ys[0, h]
        inside = np.abs(x) <= 127 * s
        assert np.all(np.abs(v[inside] - x[inside]) <= 0.5 * s * (1 + 1e-6) + np.abs(v[inside]) * 2.0 ** -8)
        top = float(oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits_rne(np.float32(127) * np.float32(s))).reshape(-1)[0])
        out = np.abs(x) >= 127.5 * s * (1 + 1e-6)
        assert out.any() or h == 3
        np.testing.assert_array_equal(v[out], np.sign(x[out]) * top)
    assert np.all(y[0, 2, :, :Dn] == 0)                           # +0 everywhere
    np.testing.assert_array_equal(y[..., Dn:], k[..., Dn:])       # RoPE part unchanged
