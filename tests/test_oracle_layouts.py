"""Pins for the oracle's float16 inputs and (B, S, H, D) layouts.

Float16: MindIE Turbo page "Attention量化", tables 1 and 2 list float16 and bfloat16 variants
of the attention quantisation; the float16 patterns are widened exactly to float32 (checked
against hand-worked values and against numpy's own binary16 type for every pattern).
Layouts: reading L4 of ``oracle.layout`` -- a (B, S, H, D) tensor is the (B, H, S, D) one with
axes 1 and 2 exchanged; every check below builds the other layout with explicit element loops,
independently of the oracle's own view.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from test_oracle_quant import _code
from test_oracle_recall import brute_by_lower_value


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _bshd_by_loops(x):
    """(B, H, S, D) -> (B, S, H, D), element by element."""
    B, H, S, D = x.shape
    y = np.empty((B, S, H, D), dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                y[b, s, h, :] = x[b, h, s, :]
    return y


def _f16_bits(rng, shape, std=1.0):
    return (rng.normal(size=shape) * std).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------- float16 values


def test_f16_widening_hand_values():
    cases = {
        0x0000: 0.0, 0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
        0x0400: 2.0 ** -14, 0x3555: 0.333251953125, 0x3800: 0.5, 0xB7FF: -(2047 / 4096), 0x7C00: math.inf,
        0xFC00: -math.inf,
    }
    got = oracle.f16_bits_to_f32(np.array(list(cases), np.uint16))
    for (bits, want), g in zip(cases.items(), got):
        assert float(g) == want, hex(bits)
    assert _u32(oracle.f16_bits_to_f32(np.array([0x8000], np.uint16)))[0] == 0x80000000  # -0.0


def test_f16_widening_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_bits_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(_u32(mine[~nan]), _u32(ref[~nan]))
    assert np.array_equal(oracle.bits16_to_f64(bits[~nan], "f16"), ref[~nan].astype(np.float64))
    with pytest.raises(ValueError):
        oracle.bits16_to_f32(bits, "f8")


# ----------------------------------------------------------------------------- calibration


@pytest.mark.parametrize("seed", range(8))
def test_f16_windows_match_brute_force(seed):
    # float16 heads with many duplicates (coarse values) against the sort-free brute force
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(8, 160))
    vals = (rng.integers(-12, 13, size=n) * rng.choice([0.125, 0.375, 1.5, 1000.0])).astype(np.float16)
    vals[rng.random(n) < 0.1] = np.float16(-0.0)
    head = oracle.f16_bits_to_f32(vals.view(np.uint16))
    for ratio in (0.5, 0.9, 0.99, 1.0):
        if int(ratio * n) < 1:
            continue
        lo, hi = oracle.recall_window(head, ratio)
        blo, bhi = brute_by_lower_value(head, ratio)
        assert _u32(lo) == _u32(blo) and _u32(hi) == _u32(bhi), (seed, ratio)


def test_bshd_calibration_equals_bhsd():
    rng = np.random.default_rng(71)
    B, H, S, D = 3, 4, 5, 8  # H != S, B > 1: an exchanged axis would mix heads
    x = (rng.standard_t(3, size=(B, H, S, D)) * np.exp(rng.uniform(-1, 1, size=(1, H, 1, 1)))).astype(np.float32)
    y = _bshd_by_loops(x)
    for ratio in (1.0, 0.9, 0.5):
        lo, hi = oracle.calibrate(x, ratio)
        lo2, hi2 = oracle.calibrate(y, ratio, layout="BSHD")
        assert np.array_equal(_u32(lo), _u32(lo2)) and np.array_equal(_u32(hi), _u32(hi2))
    # and head h of the BSHD tensor is what the calibration of head h reads
    for h in range(H):
        lo, hi = oracle.recall_window(y[:, :, h, :].reshape(-1), 0.9)
        assert _u32(lo) == _u32(oracle.calibrate(y, 0.9, layout="BSHD")[0][h])
    with pytest.raises(ValueError):
        oracle.calibrate(y, 0.9, layout="SBHD")


# ----------------------------------------------------------------------------- quantisation


def test_f16_codes_match_exact_rational_rounding():
    rng = np.random.default_rng(72)
    B, H, S, Dn, Dr = 1, 3, 24, 16, 8
    sigma = np.exp(rng.uniform(-1, 1, size=H)).astype(np.float32)
    k = (rng.normal(size=(B, H, S, Dn + Dr)) * sigma.reshape(1, H, 1, 1)).astype(np.float16).view(np.uint16)
    scale = (sigma * np.float32(2.5) / np.float32(127)).astype(np.float32)
    codes, rope = oracle.quantize_k(k, scale, Dn, dtype="f16")
    xs = k[..., :Dn].view(np.float16).astype(np.float64)
    for idx in np.ndindex(codes.shape):
        assert codes[idx] == _code(float(xs[idx]), float(scale[idx[1]])), idx
    assert np.array_equal(rope, k[..., Dn:])


def test_f16_codes_hand_values():
    # exact float16 quotients: n + 1/2 rounds to even, saturation at +-127; a zero scale gives 0
    s = np.float32(0.5)
    vals = np.array([0.25, 0.75, 1.25, -1.25, 63.25, 63.75, 100.0, -0.0], np.float16)
    k = np.concatenate([vals.view(np.uint16), np.array([0x3C00] * 8, np.uint16)]).reshape(1, 1, 1, 16)
    codes, rope = oracle.quantize_k(k, np.array([s]), 8, dtype="f16")
    assert codes.reshape(-1).tolist() == [0, 2, 2, -2, 126, 127, 127, 0]
    assert rope.reshape(-1).tolist() == [0x3C00] * 8
    codes0, _ = oracle.quantize_k(k, np.array([0.0], np.float32), 8, dtype="f16")
    assert not codes0.any()


def test_bshd_quantize_equals_bhsd():
    rng = np.random.default_rng(73)
    B, H, S, Dn, Dr = 2, 3, 5, 16, 8
    for dtype in ("bf16", "f16"):
        if dtype == "bf16":
            k = oracle.f32_to_bf16_bits_rne(rng.normal(size=(B, H, S, Dn + Dr)).astype(np.float32))
        else:
            k = _f16_bits(rng, (B, H, S, Dn + Dr))
        scale = np.exp(rng.uniform(-5, -3, size=H)).astype(np.float32)
        codes, rope = oracle.quantize_k(k, scale, Dn, dtype=dtype)
        c2, r2 = oracle.quantize_k(_bshd_by_loops(k), scale, Dn, dtype=dtype, layout="BSHD")
        assert np.array_equal(c2, _bshd_by_loops(codes)) and np.array_equal(r2, _bshd_by_loops(rope))


# ----------------------------------------------------------------------------- decode


def _sdpa(qd, kd, vd, sm):
    q = torch.from_numpy(qd).unsqueeze(2)
    return torch.nn.functional.scaled_dot_product_attention(q, torch.from_numpy(kd), torch.from_numpy(vd),
                                                            scale=float(sm)).squeeze(2).numpy()


def test_f16_decode_is_attention_over_dequantised_cache():
    rng = np.random.default_rng(74)
    B, H, T, Dn, Dr, Dv = 2, 3, 40, 32, 16, 32
    qb = _f16_bits(rng, (B, H, Dn + Dr))
    codes = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    scale = np.exp(rng.uniform(-6, -2, size=H)).astype(np.float32)
    rope = _f16_bits(rng, (B, H, T, Dr))
    vb = _f16_bits(rng, (B, H, T, Dv), std=2.0)
    sm = np.float32(1 / math.sqrt(Dn + Dr))
    out = oracle.decode_attn(qb, codes, scale, rope, vb, sm, dtype="f16")
    kd = np.concatenate([codes.astype(np.float64) * scale.astype(np.float64).reshape(1, H, 1, 1),
                         rope.view(np.float16).astype(np.float64)], axis=-1)
    ref = _sdpa(qb.view(np.float16).astype(np.float64), kd, vb.view(np.float16).astype(np.float64), sm)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_bshd_decode_and_append_equal_bhsd():
    rng = np.random.default_rng(75)
    B, H, T, Dn, Dr, Dv = 2, 3, 12, 16, 8, 16
    for dtype in ("bf16", "f16"):
        bits = (lambda shape, std=1.0: oracle.f32_to_bf16_bits_rne(
            (rng.normal(size=shape) * std).astype(np.float32))) if dtype == "bf16" else (
            lambda shape, std=1.0: _f16_bits(rng, shape, std))
        qb = bits((B, H, Dn + Dr))
        codes = rng.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
        scale = np.exp(rng.uniform(-6, -3, size=H)).astype(np.float32)
        rope, vb = bits((B, H, T, Dr)), bits((B, H, T, Dv))
        sm = np.float32(0.17)
        out = oracle.decode_attn(qb, codes, scale, rope, vb, sm, dtype=dtype)
        out2 = oracle.decode_attn(qb, _bshd_by_loops(codes), scale, _bshd_by_loops(rope), _bshd_by_loops(vb), sm,
                                  dtype=dtype, layout="BSHD")
        assert np.array_equal(out, out2)
        kn, vn = bits((B, H, Dn + Dr)), bits((B, H, Dv))
        kv_len = np.array([3, T - 1])
        o1, c1, r1, v1 = oracle.decode_append_attn(qb, kn, vn, scale, codes, rope, vb, kv_len, sm, Dn, dtype=dtype)
        o2, c2, r2, v2 = oracle.decode_append_attn(qb, kn, vn, scale, _bshd_by_loops(codes), _bshd_by_loops(rope),
                                                   _bshd_by_loops(vb), kv_len, sm, Dn, dtype=dtype, layout="BSHD")
        assert np.array_equal(o1, o2)
        assert np.array_equal(c2, _bshd_by_loops(c1)) and np.array_equal(r2, _bshd_by_loops(r1))
        assert np.array_equal(v2, _bshd_by_loops(v1))
        # the appended token: quantised with the head's scale, its K-rope and V copied at position kv_len[b]
        ccode, crope = oracle.quantize_k(kn.reshape(B, H, 1, Dn + Dr), scale, Dn, dtype=dtype)
        for b in range(B):
            p = int(kv_len[b])
            assert np.array_equal(c2[b, p], ccode[b, :, 0]) and np.array_equal(r2[b, p], crope[b, :, 0])
            assert np.array_equal(v2[b, p], vn[b])
