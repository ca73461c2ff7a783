"""Fake quantisation (fa3q_fake_quant) on the GPU: bf16 outputs bit for bit against
oracle.fake_quant, out of place and in place.

Cases: the MLA shape and shapes whose row parts do not line up with a lane, a head with
scale 0, every finite bf16 value against log-uniform scales (including scales whose
saturated value overflows bf16 and float32 to infinity), and the library's own
calibrated scales on a full Recall Window pass.
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


def _run(fa, x: torch.Tensor, scale: np.ndarray, Dn: int, name: str) -> np.ndarray:
    dev = torch.device("cuda:0")
    want = oracle.fake_quant(bits16(x), scale, Dn)
    xd = x.to(dev)
    sd = torch.from_numpy(scale).to(dev)
    log(f"fake_quant {name}: {tuple(x.shape)} Dn={Dn} out of place")
    y = fa.fa3q_fake_quant(xd, sd, Dn)
    torch.cuda.synchronize()
    assert_bits_equal(bits16(y), want, f"{name} out of place")
    assert torch.equal(xd.cpu().view(torch.int16), x.view(torch.int16)), "input changed"
    log(f"fake_quant {name}: in place")
    fa.fa3q_fake_quant(xd, sd, Dn, y=xd)
    torch.cuda.synchronize()
    assert_bits_equal(bits16(xd), want, f"{name} in place")
    return want


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
    sigma = synth.head_sigmas(H, seed=13)
    x = synth.activations(shape, sigma, outlier_frac=0.0005, outlier_mult=40.0, dtype=torch.bfloat16, seed=14)
    scale = (sigma.numpy() * np.float32(4.0) / np.float32(127.0)).astype(np.float32)
    if H > 1:
        scale[1] = 0.0
    y = _run(fa, x, scale, Dn, name)
    if H > 1:
        assert np.all(y[:, 1, :, :Dn] == 0)


def _all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_every_bf16_value_against_log_uniform_scales(fa):
    vals = _all_finite_bf16()
    n = len(vals)
    S = (n + 15) // 16
    H = 24
    rng = np.random.default_rng(15)
    x_bits = np.zeros((1, H, S * 16), np.uint16)
    for h in range(H):
        x_bits[0, h, :n] = rng.permutation(vals)
    x_bits = x_bits.reshape(1, H, S, 16)
    scale = np.exp(rng.uniform(np.log(1e-38), np.log(1e36), H)).astype(np.float32)
    scale[0] = np.float32(2.7e36)   # 127 * s overflows float32: saturated values become +-inf
    scale[1] = np.float32(2.67e36)  # 127 * s is finite in float32 and rounds to the bf16 maximum or inf
    scale[2] = np.float32(1.0)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16)
    y = _run(fa, x, scale, 16, "all_bf16")
    assert np.any(y[0, 0] == 0x7F80) and np.any(y[0, 0] == 0xFF80)


def test_calibrated_scales(fa):
    # the library's own calibration gives the scales, as in the fake-quantisation stage
    dev = torch.device("cuda:0")
    shape, Dn = (2, 8, 512, 128 + 64), 128
    sigma = synth.head_sigmas(8, seed=16)
    x = synth.activations(shape, sigma, law="t3", outlier_frac=0.001, outlier_mult=40.0, dtype=torch.bfloat16,
                          seed=17)
    lo, hi = fa.fa3q_calibrate_perhead(x[..., :Dn].contiguous().to(dev), 0.999)
    rmin = torch.empty(8, dtype=torch.float32, device=dev)
    rmax = torch.empty(8, dtype=torch.float32, device=dev)
    fa.fa3q_init_minmax(rmin, rmax)
    fa.fa3q_accumulate_minmax(rmin, rmax, lo, hi)
    scale = fa.fa3q_qparams(rmin, rmax).cpu().numpy()
    _run(fa, x, scale, Dn, "calibrated")
