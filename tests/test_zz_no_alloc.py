"""fa3q_decode_attn_noalloc against fa3q_decode_attn, through the C ABI.

The allocation-free entry point keeps the split softmax states in the library's static
device array instead of a caller workspace.  Two calls in a row, the second on a smaller
input, must each give fa3q_decode_attn's output bit for bit (same kernels, same split
plan), and stay within the decode tolerance of the float64 oracle on sampled (b, h).
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DECODE_DESIGN_TOL, DECODE_TOL, assert_bits_equal, bits16, f32, log, row_rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cache(fa, B, H, T, Dn, Dr, Dv, seed):
    sigma = synth.head_sigmas(H, seed=seed)
    k = synth.activations((B, H, T, Dn + Dr), sigma, outlier_frac=0.0005, outlier_mult=40.0, dtype=torch.bfloat16,
                          seed=seed + 1, device=DEV)
    scale = (sigma.to(DEV) * 6.0 / 127.0).contiguous()
    kq, kr = fa.fa3q_quantize_k(k, scale, Dn)
    del k
    v = synth.activations((B, H, T, Dv), sigma, dtype=torch.bfloat16, seed=seed + 2, device=DEV)
    q = synth.normal_tensor((B, H, Dn + Dr), dtype=torch.bfloat16, seed=seed + 3, device=DEV)
    return q, kq, scale, kr, v


def _noalloc(fa, q, kq, scale, kr, v, sm):
    """The new entry point called directly through ctypes (no binding logic in between)."""
    B, H, T, Dn = kq.shape
    Dr = kr.shape[-1]
    Dv = v.shape[-1]
    out = torch.full((B, H, Dv), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.lib().fa3q_decode_attn_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kq.data_ptr()), ctypes.c_void_p(scale.data_ptr()),
        ctypes.c_void_p(kr.data_ptr()), ctypes.c_void_p(v.data_ptr()), B, H, T, Dn, Dr, Dv, ctypes.c_float(sm),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.status_string(st)
    return out


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def test_noalloc_two_calls_match_workspace_entry(fa):
    Dn, Dr, Dv = 128, 64, 128
    sm = 1.0 / math.sqrt(Dn + Dr)
    # the second call is smaller: fewer pairs, shorter cache, fewer split states
    for B, H, T, seed in ((2, 32, 65536, 900), (1, 16, 8192, 910)):
        need = fa.fa3q_decode_attn_workspace_bytes(B, H, T, Dv)
        assert 0 < need <= fa._lib.FA3Q_NOALLOC_SCRATCH_BYTES
        q, kq, scale, kr, v = _cache(fa, B, H, T, Dn, Dr, Dv, seed)
        log(f"noalloc decode B={B} H={H} T={T} scratch={need}")
        got = _noalloc(fa, q, kq, scale, kr, v, sm)
        torch.cuda.synchronize()
        log(f"workspace decode B={B} H={H} T={T}")
        ref = fa.fa3q_decode_attn(q, kq, scale, kr, v, sm)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got).all())
        assert_bits_equal(f32(got), f32(ref), f"noalloc vs workspace output B={B} H={H} T={T}")
        osc = f32(scale)
        for b, h in ((0, 0), (B - 1, H - 1), (B // 2, H // 3)):
            o = oracle.decode_attn(bits16(q[b:b + 1, h:h + 1]), kq[b:b + 1, h:h + 1].cpu().numpy(), osc[h:h + 1],
                                   bits16(kr[b:b + 1, h:h + 1]), bits16(v[b:b + 1, h:h + 1]), sm)
            err = row_rel_err(got[b:b + 1, h:h + 1].cpu().numpy(), o)
            assert err <= DECODE_TOL and err <= DECODE_DESIGN_TOL, (B, H, T, b, h, err)
        del q, kq, scale, kr, v, got, ref
        torch.cuda.empty_cache()


def test_noalloc_without_splits_and_after_other_calls(fa):
    # one split (no scratch used), right after the calls above: same output as the workspace entry
    B, H, T, Dn, Dr, Dv = 16, 128, 256, 32, 16, 32
    sm = 1.0 / math.sqrt(Dn + Dr)
    assert fa.fa3q_decode_attn_workspace_bytes(B, H, T, Dv) == 0
    q, kq, scale, kr, v = _cache(fa, B, H, T, Dn, Dr, Dv, 920)
    log(f"noalloc decode, one split, B={B} H={H} T={T}")
    got = _noalloc(fa, q, kq, scale, kr, v, sm)
    ref = fa.fa3q_decode_attn(q, kq, scale, kr, v, sm)
    torch.cuda.synchronize()
    assert_bits_equal(f32(got), f32(ref), "noalloc vs workspace output, one split")
    # the binding's wrapper gives the same
    got2 = fa.fa3q_decode_attn_noalloc(q, kq, scale, kr, v, sm)
    torch.cuda.synchronize()
    assert_bits_equal(f32(got2), f32(ref), "binding wrapper output")
    # a call past the array's size is refused before anything runs
    big = (64, 128, 32768, 128)
    assert fa.fa3q_decode_attn_workspace_bytes(*big) > fa._lib.FA3Q_NOALLOC_SCRATCH_BYTES
    st = fa.lib().fa3q_decode_attn_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kq.data_ptr()), ctypes.c_void_p(scale.data_ptr()),
        ctypes.c_void_p(kr.data_ptr()), ctypes.c_void_p(v.data_ptr()), big[0], big[1], big[2], Dn, Dr, big[3],
        ctypes.c_float(sm), ctypes.c_void_p(got.data_ptr()), None)
    assert st == fa._lib.FA3Q_ERR_SCRATCH
    assert np.isfinite(f32(got)).all()
