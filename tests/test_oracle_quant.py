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
