"""K quantisation parity on the GPU: INT8 codes and RoPE bytes bit-for-bit vs the oracle.

Includes every finite bf16 value against fixed and random scales (the division, the
half-to-even rounding and the clamp are exercised on all inputs a bf16 K can hold),
exact half-integer quotients, zero-scale heads, Dr = 0 and ragged row counts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, bits16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _run(fa, k: torch.Tensor, scale: np.ndarray, Dn: int, name: str):
    dev = torch.device("cuda:0")
    log(f"quantize {name}: {tuple(k.shape)} Dn={Dn}")
    kq, kr = fa.fa3q_quantize_k(k.to(dev), torch.from_numpy(scale).to(dev), Dn)
    torch.cuda.synchronize()
    okq, okr = oracle.quantize_k(bits16(k), scale, Dn)
    assert_bits_equal(kq.cpu().numpy(), okq, f"{name} codes")
    if k.shape[-1] > Dn:
        assert_bits_equal(bits16(kr), okr, f"{name} rope")
    return okq


SHAPES = [
    ("mla", (2, 3, 130, 128 + 64), 128),
    ("tiny", (1, 4, 64, 32 + 16), 32),
    ("no_rope", (2, 2, 257, 16), 16),
    ("odd_units", (1, 5, 300, 96 + 8), 96),
    ("wide", (1, 2, 129, 256 + 24), 256),
    ("one_row", (1, 1, 1, 16 + 8), 16),
]


@pytest.mark.parametrize("name,shape,Dn", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(fa, name, shape, Dn):
    H = shape[1]
    sigma = synth.head_sigmas(H, seed=3)
    k = synth.activations(shape, sigma, outlier_frac=0.0005, outlier_mult=40.0, dtype=torch.bfloat16, seed=4)
    scale = (sigma.numpy() * np.float32(4.0) / np.float32(127.0)).astype(np.float32)
    if H > 1:
        scale[1] = 0.0  # a head with an all-zero range
    _run(fa, k, scale, Dn, name)


def _all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_every_bf16_value_against_many_scales(fa):
    vals = _all_finite_bf16()
    n = len(vals)
    S = (n + 15) // 16
    pad = np.zeros(S * 16, np.uint16)
    pad[:n] = vals
    scales = np.array([1e-38, 3e-30, 1e-6, 1e-3, 0.0123, 0.5, 1.0, 1.0 / 3.0, 3.3, 127.0, 1e10, 3e38],
                      dtype=np.float32)
    H = len(scales)
    k_bits = np.broadcast_to(pad.reshape(1, 1, S, 16), (1, H, S, 16)).copy()
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    codes = _run(fa, k, scales, 16, "all_bf16")
    assert codes.min() >= -127 and codes.max() <= 127


def test_every_bf16_value_against_random_scales(fa):
    # 64 log-uniform scales over [1e-6, 1e6]: every bf16 value lands near many half-integer
    # quotients, where a multiply by the reciprocal can round differently from the division
    vals = _all_finite_bf16()
    n = len(vals)
    S = (n + 15) // 16
    pad = np.zeros(S * 16, np.uint16)
    pad[:n] = vals
    rng = np.random.default_rng(7)
    scales = np.exp(rng.uniform(np.log(1e-6), np.log(1e6), 64)).astype(np.float32)
    H = len(scales)
    k_bits = np.broadcast_to(pad.reshape(1, 1, S, 16), (1, H, S, 16)).copy()
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    _run(fa, k, scales, 16, "all_bf16_random_scales")


def test_exact_half_integer_quotients(fa):
    s = np.float32(0.25)
    halves = (np.arange(-128, 128, dtype=np.float32) + np.float32(0.5)) * s  # 2n+1 <= 255: exact in bf16
    n = len(halves)
    S = (n + 15) // 16
    x = np.zeros(S * 16, np.float32)
    x[:n] = halves
    k_bits = oracle.f32_to_bf16_bits_rne(x).reshape(1, 1, S, 16)
    assert np.array_equal(oracle.bf16_bits_to_f32(k_bits).reshape(-1), x)
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    codes = _run(fa, k, np.array([s]), 16, "halves").reshape(-1)[:n]
    assert codes[np.argmin(np.abs(halves - 0.125))] == 0      # 0.5 -> 0 (even)
    assert codes[np.argmin(np.abs(halves - 0.375))] == 2      # 1.5 -> 2


def test_deterministic(fa):
    dev = torch.device("cuda:0")
    sigma = synth.head_sigmas(8, seed=31)
    k = synth.activations((3, 8, 200, 192), sigma, outlier_frac=0.0005, dtype=torch.bfloat16, seed=32).to(dev)
    scale = (sigma * 4 / 127).to(dev)
    a = [t.clone() for t in fa.fa3q_quantize_k(k, scale, 128)]
    b = fa.fa3q_quantize_k(k, scale, 128)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
