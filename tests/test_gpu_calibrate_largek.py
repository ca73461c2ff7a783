"""Recall Window past the on-chip tail lists: the histogram path of 16-bit inputs.

msModelSlim page "FA3量化", section 原理 -> 算法流程: the window is defined for every ratio
in (0, 1] through target_num = int(ratio*N); K = N - target_num + 1 windows.  Once K is
above fa3q_calibrate_max_windows the library counts each head into a 65536-bin histogram
and finds the window from it.  Every head is compared bit for bit with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, f32, log, oracle_windows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _k_of(ratio, N):
    return N - int(ratio * N) + 1


def _check(fa, x, ratio, what):
    B, H, S, D = x.shape
    N = B * S * D
    K = _k_of(ratio, N)
    assert K > fa.fa3q_calibrate_max_windows(x.dtype), (what, K)
    log(f"{what}: shape {tuple(x.shape)} ratio={ratio!r} K={K} ws={fa.fa3q_calibrate_workspace_bytes(x.dtype, B, H, S, D, ratio)}")
    wmin, wmax = fa.fa3q_calibrate_perhead(x, ratio)
    torch.cuda.synchronize()
    lo, hi = oracle_windows(x, ratio)
    assert_bits_equal(f32(wmin), lo, f"{what} win_min")
    assert_bits_equal(f32(wmax), hi, f"{what} win_max")
    return wmin, wmax


def test_first_k_past_the_tail_lists(fa):
    cap = fa.fa3q_calibrate_max_windows(torch.bfloat16)
    shape = (2, 8, 4096, 128)
    N = 2 * 4096 * 128
    sigma = synth.head_sigmas(8, seed=31)
    x = synth.activations(shape, sigma, law="t3", outlier_frac=1e-4, outlier_mult=60.0, dtype=torch.bfloat16,
                          seed=32, device=DEV)
    ratio = (N - cap) / N  # exact in double: t = N - cap, K = cap + 1
    assert _k_of(ratio, N) == cap + 1
    _check(fa, x, ratio, "K = cap + 1")
    for r in (0.98, 0.9, 0.5, 0.01):
        _check(fa, x, r, f"ratio {r}")


def test_config2_heads_at_0_99_and_0_9(fa):
    # a full calibration batch of the DeepSeek-like K-nope shape: 128 heads of 2,097,152 values
    shape = (8, 128, 2048, 128)
    sigma = synth.head_sigmas(128, seed=2024)
    x = synth.activations(shape, sigma, law="t3", dtype=torch.bfloat16, seed=100, device=DEV)
    for ratio, K in ((0.99, 20973), (0.9, 209717)):
        assert _k_of(ratio, 8 * 2048 * 128) == K
        _check(fa, x, ratio, f"config-2 batch ratio {ratio}")


def test_several_batches_in_one_call(fa):
    shape, ratio, nb = (4, 16, 1024, 128), 0.95, 4
    H = shape[1]
    sigma = synth.head_sigmas(H, seed=41)
    xs = [synth.activations(shape, sigma, law="t3", outlier_frac=1e-4, outlier_mult=60.0, dtype=torch.bfloat16,
                            seed=42 + b, device=DEV) for b in range(nb)]
    run_min = torch.empty(H, dtype=torch.float32, device=DEV)
    run_max = torch.empty(H, dtype=torch.float32, device=DEV)
    win_min = torch.empty((nb, H), dtype=torch.float32, device=DEV)
    win_max = torch.empty((nb, H), dtype=torch.float32, device=DEV)
    log(f"batches nb={nb} {shape} ratio={ratio} K={_k_of(ratio, 4 * 1024 * 128)}")
    fa.fa3q_calibrate_batches(xs, ratio, run_min, run_max, True, win_min, win_max)
    torch.cuda.synchronize()
    omin, omax = oracle.init_running(H)
    for b in range(nb):
        lo, hi = oracle_windows(xs[b], ratio)
        assert_bits_equal(f32(win_min[b]), lo, f"batch {b} win_min")
        assert_bits_equal(f32(win_max[b]), hi, f"batch {b} win_max")
        omin, omax = oracle.accumulate(omin, omax, lo, hi)
    assert_bits_equal(f32(run_min), omin, "run_min")
    assert_bits_equal(f32(run_max), omax, "run_max")


@pytest.mark.parametrize("S", [2048, 1024])  # two parts per head / one part that also finds the window
def test_degenerate_heads(fa, S):
    # head 0 all equal (every value in one bin: its 16-bit counters wrap many times), head 1
    # two values, head 2 signed zeros and a few values, head 3 every finite bf16 pattern (more
    # distinct values than the window search keeps on chip), head 4 arithmetic progression,
    # head 5 normal
    B, H, D = 1, 6, 512
    N = S * D
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    x = torch.empty((B, H, S, D), dtype=torch.bfloat16)
    x[0, 0] = 1.5
    x[0, 1] = torch.where(torch.rand((S, D), generator=g) < 0.3, torch.tensor(-2.0), torch.tensor(3.0)).to(torch.bfloat16)
    z = torch.where(torch.rand((S, D), generator=g) < 0.5, torch.tensor(-0.0), torch.tensor(0.0))
    z.view(-1)[:1000] = torch.randn(1000, generator=g)
    x[0, 2] = z.to(torch.bfloat16)
    bits = torch.arange(N, dtype=torch.int64) % 65536
    finite = ((bits >> 7) & 0xff) != 0xff
    pats = bits[finite]
    pats = pats[torch.randperm(pats.numel(), generator=g)]
    reps = (N + pats.numel() - 1) // pats.numel()
    x[0, 3] = pats.repeat(reps)[:N].to(torch.int16).view(torch.bfloat16).view(S, D)
    x[0, 4] = (torch.arange(N, dtype=torch.float32) % 251).to(torch.bfloat16).view(S, D)
    x[0, 5] = torch.randn((S, D), generator=g).to(torch.bfloat16)
    x = x.to(DEV)
    for ratio in (0.97, 0.5, 1.0 / N):
        _check(fa, x, ratio, f"degenerate heads ratio {ratio!r}")


def _sampled_vectors(Qv):
    """Head vectors the histogram path's bound sample reads: 32 runs of 128 vectors, one per
    1/32 of the head at a fixed phase inside it (whole 128-byte lines)."""
    stride = Qv // 32
    room = max(0, stride - 128)
    out = []
    for j in range(32):
        phase = (((((2 * j + 1) * 40503) & 0xFFFF) * room) >> 16) & ~7
        out.extend(range(j * stride + phase, j * stride + phase + 128))
    return out


def test_sample_that_misses_the_tails(fa):
    # heads whose sampled vectors all hold an extreme value the rest of the head lacks: the
    # bounds from the sample leave fewer than K values beyond them, the exact check fails and
    # the window workgroup counts the head again without bounds
    B, H, S, D = 2, 4, 4096, 256
    N = B * S * D
    Lv = S * D // 8
    ratio = 0.98
    assert _k_of(ratio, N) > 32760  # more windows than the sample holds values
    sigma = synth.head_sigmas(H, seed=51)
    x = synth.activations((B, H, S, D), sigma, law="t3", dtype=torch.bfloat16, seed=52, device=DEV)
    flat = x.view(B, H, S * D)
    for h, val in ((0, -100.0), (1, 100.0), (2, -100.0)):
        for qv in _sampled_vectors(B * Lv):
            b, w = divmod(qv, Lv)
            flat[b, h, 8 * w:8 * w + 8] = val
        if h == 2:
            flat[:, h, : S * D // 2] = 100.0  # and half the head beyond the other bound
    _check(fa, x, ratio, "sample misses the tails")


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_few_heads_many_parts(fa, layout):
    # two heads of 8.4M values: 16 parts per head (head-major) or 8 (token-major rows), whose
    # records the summing kernel adds up across many workgroups; head 0 holds one value only
    # (its counters wrap in every part), head 1 Student-t(3) values and two signed zeros
    B, H, S, D = 1, 2, 8192, 1024
    N = B * S * D
    g = torch.Generator(device="cpu")
    g.manual_seed(71)
    x = torch.empty((B, H, S, D), dtype=torch.bfloat16)
    x[0, 0] = 1.5
    sigma = synth.head_sigmas(1, seed=72)
    x[0, 1] = synth.activations((1, 1, S, D), sigma, law="t3", dtype=torch.bfloat16, seed=73)[0, 0]
    x[0, 1, 0, :2] = torch.tensor([0.0, -0.0], dtype=torch.bfloat16)
    xl = x if layout == "BHSD" else x.transpose(1, 2).contiguous()
    xl = xl.to(DEV)
    for ratio in (0.999, 0.5):
        K = _k_of(ratio, N)
        log(f"few heads many parts: {layout} ratio={ratio} K={K}")
        wmin, wmax = fa.fa3q_calibrate_ex([xl], ratio, layout=layout)
        torch.cuda.synchronize()
        lo, hi = oracle_windows(x, ratio)
        assert_bits_equal(f32(wmin[0]), lo, f"{layout} ratio {ratio} win_min")
        assert_bits_equal(f32(wmax[0]), hi, f"{layout} ratio {ratio} win_max")
