"""Decode attention with Q, K and V all per-head INT8, on the GPU against the float64 oracle.

Q, K and V are quantised on the GPU by fa3q_quantize_k (V with Dr = 0, Q as a one-token
tensor) and checked bit for bit against the oracle's quantiser; the attention output is
then compared with the oracle's attention over the dequantised tensors.  Covers the tiny
and MLA shapes, the split path, no RoPE part, and the narrowest and widest V.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DECODE_DESIGN_TOL, DECODE_TOL, bits16, log, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _scale(sigma, mult=4.0):
    return (sigma.numpy().astype(np.float32) * np.float32(mult) / np.float32(127.0)).astype(np.float32)


@pytest.mark.parametrize("name,shape", [
    ("tiny", (1, 4, 64, 32, 16, 32)),
    ("mla", (4, 16, 1024, 128, 64, 128)),
    ("splits", (2, 2, 4096, 128, 64, 128)),
    ("no_rope", (2, 8, 300, 64, 0, 64)),
    ("narrow_v", (3, 4, 129, 16, 8, 16)),
    ("wide_v", (1, 2, 200, 32, 16, 512)),
])
def test_qkv8_against_oracle(fa, name, shape):
    dev = torch.device("cuda:0")
    B, H, T, Dn, Dr, Dv = shape
    seed = 600 + sum(shape)
    sig = synth.head_sigmas(H, seed=seed)
    q = synth.activations((B, H, 1, Dn + Dr), sig, dtype=torch.bfloat16, seed=seed + 1)
    k = synth.activations((B, H, T, Dn + Dr), sig, outlier_frac=0.001, dtype=torch.bfloat16, seed=seed + 2)
    v = synth.activations((B, H, T, Dv), sig, outlier_frac=0.001, dtype=torch.bfloat16, seed=seed + 3)
    sq, sk, sv = _scale(sig, 3.0), _scale(sig, 4.0), _scale(sig, 5.0)
    log(f"qkv8 {name}: B={B} H={H} T={T} Dn={Dn} Dr={Dr} Dv={Dv}")
    t = lambda a: torch.from_numpy(a).to(dev)
    qc, qr = fa.fa3q_quantize_k(q.to(dev), t(sq), Dn)
    kc, kr = fa.fa3q_quantize_k(k.to(dev), t(sk), Dn)
    vc, _ = fa.fa3q_quantize_k(v.to(dev), t(sv), Dv)
    sm = 1.0 / math.sqrt(Dn + Dr)
    out = fa.fa3q_decode_attn_qkv8(qc.reshape(B, H, Dn), qr.reshape(B, H, Dr) if Dr else None, t(sq), kc, t(sk),
                                   kr if Dr else None, vc, t(sv), sm)
    torch.cuda.synchronize()
    # codes bit for bit against the oracle's quantiser
    oqc, oqr = oracle.quantize_k(bits16(q), sq, Dn)
    okc, okr = oracle.quantize_k(bits16(k), sk, Dn)
    ovc, _ = oracle.quantize_k(bits16(v), sv, Dv)
    np.testing.assert_array_equal(qc.cpu().numpy(), oqc)
    np.testing.assert_array_equal(kc.cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.cpu().numpy(), ovc)
    ref = oracle.decode_attn_qkv8(oqc.reshape(B, H, Dn), oqr.reshape(B, H, Dr), sq, okc, sk, okr, ovc, sv, sm)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    assert err <= DECODE_TOL, err
    assert err <= DECODE_DESIGN_TOL, err
