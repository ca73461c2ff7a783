"""Decode step with append and ragged lengths on the GPU against the float64 oracle.

The cache (capacity T) is written in place at position kv_len[b]; after each call the
whole cache is compared bit for bit with the oracle's updated cache, and the output
within the decode tolerances.  Covers appends at position 0, at split boundaries and
at the last slot, ragged lengths without an append, several splits per (b, h), the MLA
head dims, clamping of out-of-range lengths, and identity with fa3q_decode_attn when
every length is the capacity.
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


def _inputs(B, H, T, Dn, Dr, Dv, seed):
    g = np.random.default_rng(seed)
    codes = g.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    sigma = synth.head_sigmas(H, seed=seed)
    # scales as calibration would give for the synthetic K: absmax / 127 of a few sigma
    scale = (sigma.numpy().astype(np.float32) * np.float32(4.0) / np.float32(127.0)).astype(np.float32)
    rope = synth.activations((B, H, T, Dr), sigma, dtype=torch.bfloat16, seed=seed + 1)
    v = synth.activations((B, H, T, Dv), sigma, dtype=torch.bfloat16, seed=seed + 2)
    q = synth.normal_tensor((B, H, Dn + Dr), dtype=torch.bfloat16, seed=seed + 3)
    k_new = synth.activations((B, H, 1, Dn + Dr), sigma, dtype=torch.bfloat16, seed=seed + 4).reshape(B, H, Dn + Dr)
    v_new = synth.activations((B, H, 1, Dv), sigma, dtype=torch.bfloat16, seed=seed + 5).reshape(B, H, Dv)
    return q, codes, scale, rope, v, k_new.contiguous(), v_new.contiguous()


def _step(fa, name, q, codes, scale, rope, v, kv_len, k_new=None, v_new=None, oracle_len=None):
    dev = torch.device("cuda:0")
    B, H, T, Dn = codes.shape
    Dr, Dv = rope.shape[-1], v.shape[-1]
    sm = 1.0 / math.sqrt(Dn + Dr)
    log(f"decode step {name}: B={B} H={H} T={T} Dn={Dn} Dr={Dr} Dv={Dv} append={k_new is not None} "
        f"kv_len={list(kv_len)[:8]}")
    cq = torch.from_numpy(codes).to(dev)
    cr = rope.to(dev).contiguous()
    cv = v.to(dev).contiguous()
    out = fa.fa3q_decode_append_attn(q.to(dev), None if k_new is None else k_new.to(dev),
                                     None if v_new is None else v_new.to(dev), torch.from_numpy(scale).to(dev),
                                     cq, cr, cv, torch.tensor(kv_len, dtype=torch.int32, device=dev), sm)
    torch.cuda.synchronize()
    lens = np.asarray(kv_len if oracle_len is None else oracle_len, np.int64)
    ref, rc, rr, rv = oracle.decode_append_attn(bits16(q), None if k_new is None else bits16(k_new),
                                                None if v_new is None else bits16(v_new), scale, codes, bits16(rope),
                                                bits16(v), lens, sm, Dn)
    np.testing.assert_array_equal(cq.cpu().numpy(), rc)
    np.testing.assert_array_equal(bits16(cr.cpu()), rr)
    np.testing.assert_array_equal(bits16(cv.cpu()), rv)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    assert err <= DECODE_TOL, err
    assert err <= DECODE_DESIGN_TOL, err
    return got


def test_append_small_heads_every_position(fa):
    # one sequence per position 0 .. T-1 of a one-split cache
    B, H, T, Dn, Dr, Dv = 64, 4, 64, 32, 16, 32
    q, codes, scale, rope, v, kn, vn = _inputs(B, H, T, Dn, Dr, Dv, 500)
    _step(fa, "every_position", q, codes, scale, rope, v, list(range(B)), kn, vn)


def test_append_at_split_boundaries(fa):
    # few (b,h) pairs and a long cache: several splits per (b,h), combined by the combine kernel
    B, H, T, Dn, Dr, Dv = 8, 2, 2048, 128, 64, 128
    q, codes, scale, rope, v, kn, vn = _inputs(B, H, T, Dn, Dr, Dv, 510)
    ws = fa.fa3q_decode_attn_workspace_bytes(B, H, T, Dv)
    assert ws > 0  # the split path
    _step(fa, "split_boundaries", q, codes, scale, rope, v, [0, 1, 255, 256, 257, 1023, 2046, 2047], kn, vn)


def test_ragged_without_append(fa):
    B, H, T, Dn, Dr, Dv = 8, 2, 2048, 128, 64, 128
    q, codes, scale, rope, v, _, _ = _inputs(B, H, T, Dn, Dr, Dv, 520)
    _step(fa, "ragged", q, codes, scale, rope, v, [1, 2, 255, 256, 257, 1000, 2047, 2048])


def test_mla_shape_random_lengths(fa):
    B, H, T, Dn, Dr, Dv = 16, 16, 1024, 128, 64, 128
    q, codes, scale, rope, v, kn, vn = _inputs(B, H, T, Dn, Dr, Dv, 530)
    lens = np.random.default_rng(531).integers(0, T, size=B).tolist()
    _step(fa, "mla_random_lengths", q, codes, scale, rope, v, lens, kn, vn)


def test_out_of_range_lengths_are_clamped(fa):
    B, H, T, Dn, Dr, Dv = 4, 2, 512, 32, 16, 32
    q, codes, scale, rope, v, kn, vn = _inputs(B, H, T, Dn, Dr, Dv, 540)
    # append: below 0 acts as 0, at or past T as T-1
    _step(fa, "clamp_append", q, codes, scale, rope, v, [-5, 0, T, T + 100], kn, vn, oracle_len=[0, 0, T - 1, T - 1])
    # attention only: below 1 acts as 1, past T as T
    _step(fa, "clamp_ragged", q, codes, scale, rope, v, [-1, 0, T + 1, T], oracle_len=[1, 1, T, T])


def test_full_lengths_match_plain_decode_exactly(fa):
    dev = torch.device("cuda:0")
    B, H, T, Dn, Dr, Dv = 4, 8, 1500, 128, 64, 128
    q, codes, scale, rope, v, _, _ = _inputs(B, H, T, Dn, Dr, Dv, 550)
    sm = 1.0 / math.sqrt(Dn + Dr)
    args = (q.to(dev), torch.from_numpy(codes).to(dev), torch.from_numpy(scale).to(dev), rope.to(dev), v.to(dev))
    plain = fa.fa3q_decode_attn(*args, sm)
    step = fa.fa3q_decode_append_attn(args[0], None, None, args[2], args[1], args[3], args[4],
                                      torch.full((B,), T, dtype=torch.int32, device=dev), sm)
    torch.cuda.synchronize()
    assert torch.equal(plain, step)


def test_binding_rejects_half_a_token(fa):
    dev = torch.device("cuda:0")
    B, H, T, Dn, Dr, Dv = 1, 1, 8, 16, 8, 16
    q, codes, scale, rope, v, kn, vn = _inputs(B, H, T, Dn, Dr, Dv, 560)
    with pytest.raises(ValueError):
        fa.fa3q_decode_append_attn(q.to(dev), kn.to(dev), None, torch.from_numpy(scale).to(dev),
                                   torch.from_numpy(codes).to(dev), rope.to(dev), v.to(dev),
                                   torch.zeros(B, dtype=torch.int32, device=dev), 1.0)
