"""Decode step over a paged cache on the GPU against the float64 oracle.

The pools (num_pages, H, P, .) are filled by a scatter written here from a contiguous
synthetic cache, under a random page permutation with spare pages holding junk.  After
each call the pools are compared bit for bit with the oracle's pools (the append writes
one row per (b, h)), and the output within the decode tolerances.  Covers page sizes 16,
64 and 256, lengths at and around page and split boundaries, an append into an empty
cache and into the last slot, several splits per (b, h), the MLA head dims, shared pages
without an append, out-of-range table entries (clamped), and identity with
fa3q_decode_append_attn when one page holds a whole sequence.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DECODE_DESIGN_TOL, DECODE_TOL, bits16, log, row_rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _scatter(cache: torch.Tensor, page_of: np.ndarray, NP: int, P: int, junk: int) -> torch.Tensor:
    """(B,H,T,D) -> (NP,H,P,D): logical page j of sequence b at physical page page_of[b, j]."""
    B, H, T, D = cache.shape
    pool = torch.full((NP, H, P, D), junk, dtype=torch.int16 if cache.dtype != torch.int8 else torch.int8)
    src = cache.view(torch.int16) if cache.dtype == torch.bfloat16 else cache
    for b in range(B):
        for j in range(T // P):
            pool[int(page_of[b, j])] = src[b, :, j * P:(j + 1) * P]
    return pool.view(torch.bfloat16) if cache.dtype == torch.bfloat16 else pool


def _case(B, H, P, MP, Dn, Dr, Dv, seed, spare=5):
    T = MP * P
    NP = B * MP + spare
    g = np.random.default_rng(seed)
    sigma = synth.head_sigmas(H, seed=seed)
    codes = torch.from_numpy(g.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8))
    scale = (sigma.numpy().astype(np.float32) * np.float32(4.0) / np.float32(127.0)).astype(np.float32)
    rope = synth.activations((B, H, T, Dr), sigma, dtype=torch.bfloat16, seed=seed + 1)
    v = synth.activations((B, H, T, Dv), sigma, dtype=torch.bfloat16, seed=seed + 2)
    q = synth.normal_tensor((B, H, Dn + Dr), dtype=torch.bfloat16, seed=seed + 3)
    k_new = synth.activations((B, H, 1, Dn + Dr), sigma, dtype=torch.bfloat16, seed=seed + 4).reshape(B, H, Dn + Dr)
    v_new = synth.activations((B, H, 1, Dv), sigma, dtype=torch.bfloat16, seed=seed + 5).reshape(B, H, Dv)
    page_of = g.permutation(NP)[:B * MP].reshape(B, MP).astype(np.int32)
    # spare pages hold 90 (codes) and 0.5 (bf16): finite, and read only through a clamped entry
    pools = (_scatter(codes, page_of, NP, P, 0x5A), _scatter(rope, page_of, NP, P, 0x3F00),
             _scatter(v, page_of, NP, P, 0x3F00))
    return dict(q=q, scale=scale, pools=pools, page_of=page_of, k_new=k_new.contiguous(), v_new=v_new.contiguous(),
                dims=(B, H, P, MP, Dn, Dr, Dv))


def _step(fa, name, c, kv_len, append, table=None, oracle_table=None):
    B, H, P, MP, Dn, Dr, Dv = c["dims"]
    sm = 1.0 / math.sqrt(Dn + Dr)
    table = c["page_of"] if table is None else table
    log(f"paged step {name}: B={B} H={H} P={P} pages/seq={MP} Dn={Dn} Dr={Dr} Dv={Dv} append={append} "
        f"kv_len={list(kv_len)[:8]}")
    pc, pr, pv = (t.to(DEV).contiguous() for t in c["pools"])
    kn = c["k_new"].to(DEV) if append else None
    vn = c["v_new"].to(DEV) if append else None
    out = fa.fa3q_decode_paged_attn(c["q"].to(DEV), kn, vn, torch.from_numpy(c["scale"]).to(DEV), pc,
                                    pr if Dr else None, pv, torch.from_numpy(np.ascontiguousarray(table)).to(DEV),
                                    torch.tensor(kv_len, dtype=torch.int32, device=DEV), sm)
    torch.cuda.synchronize()
    ref, rc, rr, rv = oracle.decode_paged_attn(
        bits16(c["q"]), bits16(c["k_new"]) if append else None, bits16(c["v_new"]) if append else None, c["scale"],
        c["pools"][0].numpy(), bits16(c["pools"][1]), bits16(c["pools"][2]),
        table if oracle_table is None else oracle_table, np.asarray(kv_len, np.int64), sm, Dn)
    np.testing.assert_array_equal(pc.cpu().numpy(), rc)
    np.testing.assert_array_equal(bits16(pr.cpu()), rr)
    np.testing.assert_array_equal(bits16(pv.cpu()), rv)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = row_rel_err(got, ref)
    assert err <= DECODE_TOL, err
    assert err <= DECODE_DESIGN_TOL, err
    return out


@pytest.mark.parametrize("P", [16, 64, 256])
def test_lengths_around_page_boundaries(fa, P):
    B, H, MP, Dn, Dr, Dv = 8, 2, 4, 32, 16, 32
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=600 + P)
    T = MP * P
    appends = [0, 1, P - 1, P, P + 1, 2 * P - 1, T - 2, T - 1]
    _step(fa, f"append_P{P}", c, appends, True)
    reads = [1, 2, P - 1, P, P + 1, 3 * P, T - 1, T]
    _step(fa, f"read_P{P}", c, reads, False)


def test_several_splits_per_sequence(fa):
    # few (b,h) pairs over 4096 tokens: 256-token splits crossing 64-token pages
    B, H, P, MP, Dn, Dr, Dv = 2, 2, 64, 64, 32, 16, 32
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=610)
    _step(fa, "splits_append", c, [4095, 1000], True)
    _step(fa, "splits_read", c, [4096, 257], False)


def test_mla_dims(fa):
    B, H, P, MP, Dn, Dr, Dv = 4, 16, 64, 8, 128, 64, 128
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=620)
    _step(fa, "mla", c, [5, 64, 300, 511], True)


def test_widest_values_and_one_page_sequences(fa):
    # Dv = 512 (64 lanes per token), pages of 16 tokens, one page per sequence
    B, H, P, MP, Dn, Dr, Dv = 3, 2, 16, 1, 32, 16, 512
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=635)
    _step(fa, "wide_v_append", c, [0, 7, 15], True)
    _step(fa, "wide_v_read", c, [1, 9, 16], False)


def test_no_rope_part(fa):
    B, H, P, MP, Dn, Dr, Dv = 3, 4, 16, 5, 64, 0, 64
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=630)
    _step(fa, "no_rope", c, [0, 33, 79], True)


def test_shared_pages_without_append(fa):
    B, H, P, MP, Dn, Dr, Dv = 4, 2, 16, 3, 32, 16, 32
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=640)
    table = np.repeat(c["page_of"][:1], B, axis=0)  # every sequence reads sequence 0's pages
    c["q"][2] = c["q"][0]
    out = _step(fa, "shared", c, [48, 20, 48, 1], False, table=table)
    assert torch.equal(out[2], out[0])


def test_out_of_range_table_entries_are_clamped(fa):
    B, H, P, MP, Dn, Dr, Dv = 2, 2, 16, 4, 32, 16, 32
    c = _case(B, H, P, MP, Dn, Dr, Dv, seed=650)
    NP = c["pools"][0].shape[0]
    table = c["page_of"].copy()
    table[0, 1] = -3          # read as page 0
    table[1, 2] = NP + 40     # read as the last page
    clamped = np.clip(table, 0, NP - 1)
    _step(fa, "clamped", c, [40, 50], False, table=table, oracle_table=clamped)


def test_one_page_per_sequence_is_the_contiguous_step(fa):
    # with P = T and page b for sequence b the pools are the (B,H,T,.) cache itself: same
    # split plan and arithmetic, so the output and the written rows equal fa3q_decode_append_attn's
    B, H, T, Dn, Dr, Dv = 3, 4, 1024, 32, 16, 32
    c = _case(B, H, T, 1, Dn, Dr, Dv, seed=660, spare=0)
    table = np.arange(B, dtype=np.int32).reshape(B, 1)
    # page b <- sequence b's page: the pools are then (B,H,T,.) caches
    pools = [torch.stack([c["pools"][t][int(c["page_of"][b, 0])] for b in range(B)]).to(DEV) for t in range(3)]
    cache = [p.clone() for p in pools]
    kv_len = torch.tensor([0, 511, 1023], dtype=torch.int32, device=DEV)
    q, s = c["q"].to(DEV), torch.from_numpy(c["scale"]).to(DEV)
    kn, vn = c["k_new"].to(DEV), c["v_new"].to(DEV)
    sm = 1.0 / math.sqrt(Dn + Dr)
    log("paged step one_page_per_sequence vs fa3q_decode_append_attn")
    a = fa.fa3q_decode_paged_attn(q, kn, vn, s, pools[0], pools[1], pools[2], torch.from_numpy(table).to(DEV),
                                  kv_len, sm)
    b = fa.fa3q_decode_append_attn(q, kn, vn, s, cache[0], cache[1], cache[2], kv_len, sm)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for x, y in zip(pools, cache):
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y)
