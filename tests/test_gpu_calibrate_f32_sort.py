"""Recall Window of float32 heads past the on-chip tail lists, and of float32 (B,S,H,D) input.

(B,S,H,D) rows whose D is a power of two take the tail lists while K is within their cap
(the same sampled bounds and chunk lists as (B,H,S,D) slabs, the rows addressed one by one);
other (B,S,H,D) input and larger K take the collect-and-sort path.  The cases below cover both.

msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程: the
window is defined for every ratio in (0, 1] through target_num = int(ratio*N), K = N -
target_num + 1 windows per head.  For float32 heads with K above
fa3q_calibrate_max_windows(float32), and for float32 (B,S,H,D) input at any K, the library
collects each head's two tails through a histogram of the values' leading 16 bits, sorts them
and scans the K windows.  Every head's window is compared bit for bit with the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, log, parallel

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _k_of(ratio, N):
    return N - int(ratio * N) + 1


def _oracle(x: torch.Tensor, ratio: float, layout: str):
    heads = oracle.per_head_view(oracle.to_bhsd(x.detach().cpu().numpy(), layout))
    res = parallel(lambda h: oracle.recall_window(heads[h], ratio), range(heads.shape[0]))
    return np.array([r[0] for r in res], np.float32), np.array([r[1] for r in res], np.float32)


def _sort_path(fa, shape_bhsd, ratio, layout="BHSD"):
    """Host-side plan fact: the call takes the collect-and-sort path (two key lists of N words
    per head in the workspace, whatever the number of batches)."""
    B, H, S, D = shape_bhsd
    N = B * S * D
    ws1 = fa.fa3q_calibrate_ex_workspace_bytes(torch.float32, layout, 1, B, H, S, D, ratio)
    ws3 = fa.fa3q_calibrate_ex_workspace_bytes(torch.float32, layout, 3, B, H, S, D, ratio)
    return ws1 >= 2 * H * N * 4 and ws3 - ws1 < 4096  # only the extra windows grow with nb


def _takes_tail_lists(fa, shape_bhsd, ratio, layout):
    """(B,S,H,D) float32 rows with D a power of two and K within the tail lists' cap take the
    tail lists (one pass, sampled bounds) instead of the collect-and-sort path."""
    B, H, S, D = shape_bhsd
    K = _k_of(ratio, B * S * D)
    return layout == "BSHD" and D & (D - 1) == 0 and K <= fa.fa3q_calibrate_max_windows(torch.float32)


def _check(fa, x, ratio, what, layout="BHSD"):
    shape = tuple(x.shape) if layout == "BHSD" else (x.shape[0], x.shape[2], x.shape[1], x.shape[3])
    B, H, S, D = shape
    N = B * S * D
    K = _k_of(ratio, N)
    assert _sort_path(fa, shape, ratio, layout) != _takes_tail_lists(fa, shape, ratio, layout), (what, K)
    log(f"f32 {what}: {layout} {tuple(x.shape)} ratio={ratio!r} K={K}")
    wmin, wmax = fa.fa3q_calibrate_ex([x], ratio, layout=layout)
    torch.cuda.synchronize()
    lo, hi = _oracle(x, ratio, layout)
    assert_bits_equal(wmin[0].cpu().numpy(), lo, f"{what} win_min")
    assert_bits_equal(wmax[0].cpu().numpy(), hi, f"{what} win_max")


def _acts(shape, seed, outliers=True):
    B, H, S, D = shape
    sigma = synth.head_sigmas(H, seed=seed)
    return synth.activations(shape, sigma, law="t3", outlier_frac=1e-4 if outliers else 0.0, outlier_mult=60.0,
                             dtype=torch.float32, seed=seed + 1)


def test_first_k_past_the_tail_lists(fa):
    cap = fa.fa3q_calibrate_max_windows(torch.float32)
    shape = (2, 4, 2048, 128)
    N = 2 * 2048 * 128
    x = _acts(shape, 61).to(DEV)
    ratio = (N - cap) / N  # exact in double: t = N - cap, K = cap + 1
    assert _k_of(ratio, N) == cap + 1 == 7476
    _check(fa, x, ratio, "K = cap + 1")
    # the same heads just inside the cap take the tail lists and agree with the oracle too
    r_in = (N - cap + 1) / N
    assert _k_of(r_in, N) == cap and not _sort_path(fa, shape, r_in)
    wmin, wmax = fa.fa3q_calibrate_perhead(x, r_in)
    lo, hi = _oracle(x, r_in, "BHSD")
    assert_bits_equal(wmin.cpu().numpy(), lo, "K = cap win_min")
    assert_bits_equal(wmax.cpu().numpy(), hi, "K = cap win_max")


def test_about_100k_windows_and_overlapping_tails(fa):
    shape = (2, 8, 4096, 128)
    N = 2 * 4096 * 128
    x = _acts(shape, 71).to(DEV)
    assert _k_of(0.9, N) == 104859
    # 0.9: two separate tails; 0.5: the tails overlap (every value collected); 1/N: K = N
    for ratio in (0.9, 0.5, 1.0 / N):
        _check(fa, x, ratio, f"ratio {ratio!r}")


def test_config2_batch_at_0_99_and_0_9(fa):
    # one float32 calibration batch of the DeepSeek-like K-nope shape: 128 heads of 2,097,152 values
    shape = (8, 128, 2048, 128)
    sigma = synth.head_sigmas(128, seed=2024)
    x = synth.activations(shape, sigma, law="t3", dtype=torch.float32, seed=100, device=DEV)
    for ratio, K in ((0.99, 20973), (0.9, 209717)):
        assert _k_of(ratio, 8 * 2048 * 128) == K
        _check(fa, x, ratio, f"config-2 batch ratio {ratio}")


def test_degenerate_heads(fa):
    # head 0 all equal (one leading key, counters that wrap), head 1 two values, head 2 signed
    # zeros and a few values, head 3 every value in one leading key [1, 1 + 2^-8) (all collected,
    # sorted by the low bits alone), head 4 an arithmetic progression (many ties), head 5
    # normal, head 6 magnitudes from subnormal to 1e30 of both signs
    B, H, S, D = 1, 7, 1024, 512
    N = S * D
    g = torch.Generator(device="cpu")
    g.manual_seed(17)
    x = torch.empty((B, H, S, D), dtype=torch.float32)
    x[0, 0] = 1.5
    x[0, 1] = torch.where(torch.rand((S, D), generator=g) < 0.3, torch.tensor(-2.0), torch.tensor(3.0))
    z = torch.where(torch.rand((S, D), generator=g) < 0.5, torch.tensor(-0.0), torch.tensor(0.0))
    z.view(-1)[:1000] = torch.randn(1000, generator=g)
    x[0, 2] = z
    x[0, 3] = 1.0 + torch.rand((S, D), generator=g) * 2.0 ** -8
    x[0, 4] = (torch.arange(N, dtype=torch.float32) % 251).view(S, D)
    x[0, 5] = torch.randn((S, D), generator=g)
    e = torch.randint(-140, 100, (S, D), generator=g).to(torch.float32)
    x[0, 6] = torch.sign(torch.randn((S, D), generator=g)) * torch.exp2(e) * (1 + torch.rand((S, D), generator=g))
    x = x.to(DEV)
    for ratio in (0.97, 0.5, 1.0 / N):
        _check(fa, x, ratio, f"degenerate heads ratio {ratio!r}")


BSHD_CASES = [
    # (what, (B,H,S,D) head-major, ratios): the tail lists over rows (D a power of two, K within
    # the cap), else collect and sort
    ("rows of 32 vectors", (2, 8, 2048, 128), (0.9999, 0.99)),
    ("rows of 1 vector", (3, 5, 777, 4), (0.5, 0.999)),
    ("rows of 48 vectors", (1, 4, 1000, 192), (0.9,)),
    ("two heads, many parts", (2, 2, 8192, 128), (0.999, 0.95)),
    ("rows longer than a workgroup round", (2, 3, 64, 8192), (0.99,)),
]


@pytest.mark.parametrize("case", BSHD_CASES, ids=[c[0] for c in BSHD_CASES])
def test_bshd(fa, case):
    what, shape, ratios = case
    x = _acts(shape, 80 + len(what)).transpose(1, 2).contiguous().to(DEV)
    for ratio in ratios:
        _check(fa, x, ratio, f"BSHD {what}", layout="BSHD")


def test_one_head_in_many_parts(fa):
    # a single head of 16.8M values: the counting and collecting passes split it over 32
    # workgroups, the sorting passes over the most blocks a head gets
    shape = (4, 1, 8192, 512)
    x = _acts(shape, 91).to(DEV)
    for ratio in (0.999, 0.9):
        _check(fa, x, ratio, f"one head ratio {ratio}")


def test_batches_with_running_statistics(fa):
    # three batches through one workspace region (one batch after the other), windows and the
    # running min/max against the oracle's accumulate
    shape, nb = (2, 16, 1024, 128), 3
    H, N = shape[1], 2 * 1024 * 128
    ratio = 0.95
    assert _k_of(ratio, N) > fa.fa3q_calibrate_max_windows(torch.float32)
    xs = [_acts(shape, 120 + b).to(DEV) for b in range(nb)]
    run_min = torch.empty(H, dtype=torch.float32, device=DEV)
    run_max = torch.empty(H, dtype=torch.float32, device=DEV)
    win_min = torch.empty((nb, H), dtype=torch.float32, device=DEV)
    win_max = torch.empty((nb, H), dtype=torch.float32, device=DEV)
    log(f"f32 batches nb={nb} {shape} ratio={ratio}")
    fa.fa3q_calibrate_batches(xs, ratio, run_min, run_max, True, win_min, win_max)
    torch.cuda.synchronize()
    omin, omax = oracle.init_running(H)
    for b in range(nb):
        lo, hi = _oracle(xs[b], ratio, "BHSD")
        assert_bits_equal(win_min[b].cpu().numpy(), lo, f"batch {b} win_min")
        assert_bits_equal(win_max[b].cpu().numpy(), hi, f"batch {b} win_max")
        omin, omax = oracle.accumulate(omin, omax, lo, hi)
    assert_bits_equal(run_min.cpu().numpy(), omin, "run_min")
    assert_bits_equal(run_max.cpu().numpy(), omax, "run_max")
    # the same batches in (B,S,H,D) give the same windows
    xt = [x.transpose(1, 2).contiguous() for x in xs]
    wmin2, wmax2 = fa.fa3q_calibrate_ex(xt, ratio, layout="BSHD")
    assert_bits_equal(wmin2.cpu().numpy(), win_min.cpu().numpy(), "BSHD vs BHSD win_min")
    assert_bits_equal(wmax2.cpu().numpy(), win_max.cpu().numpy(), "BSHD vs BHSD win_max")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_tiny_heads_every_ratio(fa, dtype):
    # (B,S,H,D) heads of 4 to 24 values, every target count t = 1 .. N: lists far shorter than
    # one sort tile (float32) or one histogram part (16-bit), K = N down to 1, heads of one
    # repeated value, and a head with signed zeros
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    D = 4 if dtype == torch.float32 else 8
    for B, S, H in ((1, 1, 3), (2, 3, 2), (1, 3, 5)):
        N = B * S * D
        x = torch.randn((B, S, H, D), generator=g).to(dtype)
        x[:, :, 0, :] = 0.75                      # head 0: one value
        if H > 2:
            x[:, :, 2, :] = torch.tensor([0.0, -0.0] * (D // 2)).to(dtype)
        xd = x.to(DEV)
        for t in range(1, N + 1):
            ratio = (t + 0.5) / N if t < N else 1.0  # int(ratio * N) == t
            assert int(ratio * N) == t
            wmin, wmax = fa.fa3q_calibrate_ex([xd], ratio, layout="BSHD")
            lo, hi = _oracle(x.float() if dtype != torch.float32 else x, ratio, "BSHD")
            assert_bits_equal(wmin[0].cpu().numpy(), lo, f"{dtype} {(B, S, H, D)} t={t} win_min")
            assert_bits_equal(wmax[0].cpu().numpy(), hi, f"{dtype} {(B, S, H, D)} t={t} win_max")


def _row_run_starts(q_vecs: int, dv: int) -> list:
    """First vector of each of the 32 sample runs over (B,S,H,D) rows of dv vectors: runs of 256
    vectors, run j inside [j * stride, (j + 1) * stride) at a fixed phase, strides and phases
    whole rows."""
    stride = max(256, q_vecs // 32)
    stride = (stride + dv - 1) // dv * dv
    out = []
    for j in range(32):
        phase = ((((2 * j + 1) * 40503) & 0xFFFF) * max(0, stride - 256)) >> 16 & ~7
        out.append(j * stride + phase // dv * dv)
    return out


def test_bshd_rows_estimated_bound_that_fails_is_redone_exactly(fa):
    # (B,S,H,D) float32 rows of 128 values on the tail lists: K = 5244 against 2048 sampled
    # groups, so the head bound is an estimate checked by the merge.  Values planted where the
    # row-aligned sample reads (a group is a thread's vectors of four consecutive runs) give
    # every group an extreme: the sample bounds tightly while the head holds only 2048 values
    # beyond the bound, the check fails and the head is redone without a bound, rows addressed
    # one by one in both passes.
    dev = torch.device("cuda:0")
    B, S, H, D = 1, 8192, 2, 128
    vec, dv = 4, 128 // 4
    N = B * S * D
    ratio = 0.995
    assert _k_of(ratio, N) == 5244 <= fa.fa3q_calibrate_max_windows(torch.float32)
    rng = np.random.default_rng(29)
    x = np.ones((B, S, H, D), np.float32)
    x[:, :, 1, :] = rng.standard_normal((B, S, D)).astype(np.float32)
    starts = _row_run_starts(B * S * dv, dv)
    for g in range(8):
        lo_run, hi_run = starts[4 * g], starts[4 * g + 1]
        for t in range(256):
            for run, head, off, val in ((lo_run, 0, 0, -7.0), (hi_run, 0, 0, 9.0), (lo_run, 1, 3, -50.0)):
                row, cv = divmod(run + t, dv)
                b, s = divmod(row, S)
                x[b, s, head, cv * vec + off] = val   # head 0: both sides fail; head 1: the low side
    xt = torch.from_numpy(x).to(dev)
    assert not _sort_path(fa, (B, H, S, D), ratio, "BSHD")
    nbytes = fa.fa3q_calibrate_ex_workspace_bytes(torch.float32, "BSHD", 1, B, H, S, D, ratio)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    log(f"f32 BSHD rows, failing estimate: {tuple(xt.shape)} ratio={ratio}")
    wmin, wmax = fa.fa3q_calibrate_ex([xt], ratio, layout="BSHD", workspace=ws)
    torch.cuda.synchronize()
    lo, hi = _oracle(xt, ratio, "BSHD")
    assert_bits_equal(wmin[0].cpu().numpy(), lo, "failing estimate win_min")
    assert_bits_equal(wmax[0].cpu().numpy(), hi, "failing estimate win_max")
    # the check flags (the 256-byte block before the windows' block: low side of each head,
    # then high side): both sides of head 0, the low side of head 1
    flags = ws[nbytes - 512:nbytes - 512 + 4 * 2 * H].cpu().view(torch.int32).numpy().tolist()
    assert flags == [1, 1, 1, 0], flags
    for r in (0.999, 0.9999):
        _check(fa, xt, r, f"planted rows ratio {r}", layout="BSHD")


def _random_bshd_cases(n: int, seed: int):
    """Seeded float32 (B,S,H,D) shapes: row widths from one vector to 512 values (powers of
    two on the tail lists, 12 and 96 on collect and sort), ratios on both sides of the tail
    lists' cap."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([4, 8, 12, 16, 32, 64, 96, 128, 256, 512]))
        H = int(rng.integers(1, 7))
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 1 + 200000 // (B * D)))
        r = float(rng.choice([0.5, 0.9, 0.99, 0.999, 0.9999, 1.0]))
        cases.append((B, H, S, D, r, 500 + i))
    return cases


@pytest.mark.parametrize("B,H,S,D,ratio,seed", _random_bshd_cases(16, 777))
def test_bshd_random_shapes(fa, B, H, S, D, ratio, seed):
    N = B * S * D
    if int(ratio * N) < 1:
        pytest.skip("t = int(ratio * N) < 1")
    x = _acts((B, H, S, D), seed).transpose(1, 2).contiguous().to(DEV)
    tail = _takes_tail_lists(fa, (B, H, S, D), ratio, "BSHD")
    log(f"f32 BSHD random: {(B, S, H, D)} ratio={ratio} K={_k_of(ratio, N)} {'tail lists' if tail else 'collect and sort'}")
    wmin, wmax = fa.fa3q_calibrate_ex([x], ratio, layout="BSHD")
    torch.cuda.synchronize()
    lo, hi = _oracle(x, ratio, "BSHD")
    assert_bits_equal(wmin[0].cpu().numpy(), lo, f"random BSHD {(B, S, H, D)} win_min")
    assert_bits_equal(wmax[0].cpu().numpy(), hi, f"random BSHD {(B, S, H, D)} win_max")
