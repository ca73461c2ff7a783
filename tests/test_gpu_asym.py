"""Asymmetric per-(head, dim) K cache on the GPU against the oracle.

fa3q_quantize_asym: INT8 codes and RoPE bytes bit for bit against oracle.quantize_asym,
with bfloat16 and float16 tables, the MLA shape and shapes whose 16-byte units do not
line up with a lane (the per-vector table path), every finite bf16 value against random
per-dim scales and offsets, exact ties of x/s + o, large quotients cancelled by large
offsets, scales the fast path hands to the division (zero, tiny, huge) and saturation.
fa3q_decode_attn_asym: attention over the GPU's codes against oracle.decode_attn_asym.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DECODE_DESIGN_TOL, DECODE_TOL, assert_bits_equal, bits16, log, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _tbits(t: torch.Tensor) -> np.ndarray:
    """16-bit table (bf16 or float16) -> uint16 patterns on the host."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _dt(t: torch.Tensor) -> str:
    return "bfloat16" if t.dtype == torch.bfloat16 else "float16"


def _tables(H: int, Dn: int, sigma: torch.Tensor, dtype, seed: int, off_range: float = 40.0):
    """Per-(head, dim) scales around sigma[h]*4/127 and offsets in [-off_range, off_range]."""
    g = np.random.default_rng(seed)
    jitter = np.exp(g.uniform(np.log(0.5), np.log(2.0), (H, Dn)))
    s = sigma.numpy().astype(np.float64)[:, None] * 4.0 / 127.0 * jitter
    o = g.uniform(-off_range, off_range, (H, Dn))
    return torch.from_numpy(s).to(dtype), torch.from_numpy(o).to(dtype)


def _run(fa, k: torch.Tensor, scale: torch.Tensor, offset: torch.Tensor, Dn: int, name: str) -> np.ndarray:
    dev = torch.device("cuda:0")
    log(f"quantize_asym {name}: {tuple(k.shape)} Dn={Dn} tables={_dt(scale)}")
    kq, kr = fa.fa3q_quantize_asym(k.to(dev), scale.to(dev), offset.to(dev), Dn)
    torch.cuda.synchronize()
    okq, okr = oracle.quantize_asym(bits16(k), _tbits(scale), _tbits(offset), Dn, _dt(scale))
    assert_bits_equal(kq.cpu().numpy(), okq, f"{name} codes")
    if k.shape[-1] > Dn:
        assert_bits_equal(bits16(kr), okr, f"{name} rope")
    return okq


SHAPES = [
    ("mla", (2, 3, 130, 128 + 64), 128),
    ("tiny", (1, 4, 64, 32 + 16), 32),
    ("no_rope", (2, 2, 257, 16), 16),
    ("odd_units", (1, 5, 300, 96 + 8), 96),     # 12 units per row: tables per vector
    ("wide", (1, 2, 129, 256 + 24), 256),
    ("one_row", (1, 1, 1, 16 + 8), 16),
]


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("name,shape,Dn", SHAPES, ids=[s[0] for s in SHAPES])
def test_shapes(fa, name, shape, Dn, tdtype):
    H = shape[1]
    sigma = synth.head_sigmas(H, seed=41)
    k = synth.activations(shape, sigma, outlier_frac=0.0005, outlier_mult=40.0, dtype=torch.bfloat16, seed=42)
    scale, offset = _tables(H, Dn, sigma, tdtype, seed=43)
    scale[0, 3] = 0.0                    # a channel with an empty range
    scale[H - 1, Dn - 1] = -scale[H - 1, Dn - 1]  # a negative scale divides like any other
    codes = _run(fa, k, scale, offset, Dn, name)
    assert np.all(codes[:, 0, :, 3] == 0)


def _all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_every_bf16_value_against_random_tables(fa, tdtype):
    # each head sees every finite bf16 value, shuffled so that each value meets several of
    # the head's 16 (scale, offset) pairs; log-uniform scales put values on both sides of
    # every half-integer of x/s + o and far into saturation
    vals = _all_finite_bf16()
    n = len(vals)
    S = (n + 15) // 16
    H = 32
    rng = np.random.default_rng(11)
    k_bits = np.zeros((1, H, S * 16), np.uint16)
    for h in range(H):
        k_bits[0, h, :n] = rng.permutation(vals)
    k_bits = k_bits.reshape(1, H, S, 16)
    lo, hi = (1e-6, 1e6) if tdtype == torch.bfloat16 else (1e-7, 6e4)
    s = np.exp(rng.uniform(np.log(lo), np.log(hi), (H, 16)))
    o = rng.uniform(-300.0, 300.0, (H, 16))
    o[::2] = np.round(o[::2])                      # integer offsets on half the heads
    scale, offset = torch.from_numpy(s).to(tdtype), torch.from_numpy(o).to(tdtype)
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    codes = _run(fa, k, scale, offset, 16, f"all_bf16_{_dt(scale)}")
    assert codes.min() == -128 and codes.max() == 127


def test_exact_ties_round_half_to_even(fa):
    # x = n * 0.25 with scale 0.25 gives x/s = n exactly; offset 0.5 puts every sum on a tie
    n = np.arange(-140, 140, dtype=np.float32)
    x = n * np.float32(0.25)
    S = (len(x) + 15) // 16
    xs = np.zeros(S * 16, np.float32)
    xs[:len(x)] = x
    k_bits = oracle.f32_to_bf16_bits_rne(xs).reshape(1, 1, S, 16)
    assert np.array_equal(oracle.bf16_bits_to_f32(k_bits).reshape(-1), xs)
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    scale = torch.full((1, 16), 0.25, dtype=torch.bfloat16)
    offset = torch.full((1, 16), 0.5, dtype=torch.bfloat16)
    codes = _run(fa, k, scale, offset, 16, "ties").reshape(-1)[:len(x)]
    want = np.clip(np.where(n % 2 == 0, n, n + 1), -128, 127)  # n + 0.5 -> the even neighbour
    np.testing.assert_array_equal(codes, want.astype(np.int8))


def test_large_quotients_cancelled_by_large_offsets(fa):
    # per channel, x stays within one bf16 step of a centre c with |c/s| near 2e4, and the
    # offset is -c/s rounded to bf16: the sums land in and around the code range while the
    # reciprocal's error at that magnitude (|x/s| * 2^-22) is far above 2^-15
    H, Dn, S = 8, 64, 256
    g = np.random.default_rng(5)
    s = np.exp(g.uniform(np.log(5e-4), np.log(2e-3), (H, Dn)))
    scale = torch.from_numpy(s).to(torch.bfloat16)
    sv = scale.float().numpy().astype(np.float64)
    c = g.uniform(17.0, 31.0, (H, Dn)) * np.where(np.arange(H) % 2 == 0, 1.0, -1.0)[:, None]
    c = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits_rne(c.astype(np.float32))).astype(np.float64)
    x = c[None, :, None, :] + 0.125 * g.integers(-1, 2, (1, H, S, Dn))
    k_bits = oracle.f32_to_bf16_bits_rne(x.astype(np.float32))
    offset = torch.from_numpy(-c / sv).to(torch.bfloat16)
    k = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16)
    codes = _run(fa, k, scale, offset, Dn, "cancel")
    inside = np.abs(codes.astype(np.int32)) < 127
    assert inside.mean() > 0.1      # the cancellation is exercised, not only saturation


def test_scales_outside_the_fast_range(fa):
    # bf16 scales below 2^-100 and above 2^100 (and 0) take the correctly rounded division
    H, Dn, S = 2, 16, 64
    sigma = synth.head_sigmas(H, seed=61)
    k = synth.activations((1, H, S, Dn + 8), sigma, dtype=torch.bfloat16, seed=62)
    s = np.array([[1e-35, 1e-31, 2.0 ** -101, 2.0 ** -99, 1e30, 2.0 ** 101, 2.0 ** 99, 0.0,
                   1e-38, 3e38, 1.0, 0.01, 7e-31, 4e31, 2.0 ** -100, 2.0 ** 100]] * H, dtype=np.float64)
    o = np.linspace(-3.0, 3.0, H * Dn).reshape(H, Dn)
    _run(fa, k, torch.from_numpy(s).to(torch.bfloat16), torch.from_numpy(o).to(torch.bfloat16), Dn, "extreme_scales")


@pytest.mark.parametrize("tdtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("name,shape", [
    ("tiny", (1, 4, 64, 32, 16, 32)),
    ("mla", (4, 16, 1024, 128, 64, 128)),
    ("splits", (2, 2, 4096, 128, 64, 128)),
    ("no_rope", (2, 8, 300, 64, 0, 64)),
    ("ragged", (3, 4, 129, 16, 8, 16)),
])
def test_decode_asym_against_oracle(fa, name, shape, tdtype):
    dev = torch.device("cuda:0")
    B, H, T, Dn, Dr, Dv = shape
    seed = 700 + sum(shape)
    sig = synth.head_sigmas(H, seed=seed)
    q = synth.activations((B, H, 1, Dn + Dr), sig, dtype=torch.bfloat16, seed=seed + 1).reshape(B, H, Dn + Dr)
    k = synth.activations((B, H, T, Dn + Dr), sig, outlier_frac=0.001, dtype=torch.bfloat16, seed=seed + 2)
    v = synth.activations((B, H, T, Dv), sig, dtype=torch.bfloat16, seed=seed + 3)
    scale, offset = _tables(H, Dn, sig, tdtype, seed=seed + 4)
    log(f"decode_asym {name}: B={B} H={H} T={T} Dn={Dn} Dr={Dr} Dv={Dv} tables={_dt(scale)}")
    kc, kr = fa.fa3q_quantize_asym(k.to(dev), scale.to(dev), offset.to(dev), Dn)
    sm = 1.0 / math.sqrt(Dn + Dr)
    out = fa.fa3q_decode_attn_asym(q.to(dev), kc, scale.to(dev), offset.to(dev), kr if Dr else None, v.to(dev), sm)
    torch.cuda.synchronize()
    okc, okr = oracle.quantize_asym(bits16(k), _tbits(scale), _tbits(offset), Dn, _dt(scale))
    assert_bits_equal(kc.cpu().numpy(), okc, f"{name} codes")
    ref = oracle.decode_attn_asym(bits16(q), okc, _tbits(scale), _tbits(offset), okr, bits16(v), sm, _dt(scale))
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    assert err <= DECODE_TOL, err
    assert err <= DECODE_DESIGN_TOL, err
