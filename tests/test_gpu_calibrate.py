"""Calibration parity on the GPU: every head's window bit-for-bit against the oracle.

Covers float32 and bf16 inputs, several chunks per slab and ragged chunk tails,
K from 1 to 4196 windows, heavy ties (coarse values), signed zeros, constant heads,
monotone heads in ascending and descending memory order (the latter makes every
streamed value a new extreme), and the accumulate/qparams stages over batches.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_bits_equal, f32, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _host_f32(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().to(torch.float32).numpy()


def _check(fa, x: torch.Tensor, ratios, name):
    dev = torch.device("cuda:0")
    xg = x.to(dev)
    xf = _host_f32(x)
    for ratio in ratios:
        N = x.shape[0] * x.shape[2] * x.shape[3]
        K = N - int(ratio * N) + 1
        log(f"calibrate {name}: {x.dtype} {tuple(x.shape)} ratio={ratio} K={K}")
        wmin, wmax = fa.fa3q_calibrate_perhead(xg, ratio)
        torch.cuda.synchronize()
        omin, omax = oracle.calibrate(xf, ratio)
        assert_bits_equal(f32(wmin), omin, f"{name} win_min ratio={ratio}")
        assert_bits_equal(f32(wmax), omax, f"{name} win_max ratio={ratio}")


RANDOM_CASES = [
    # name, dtype, (B, H, S, D), law, ratios
    ("f32_ragged", torch.float32, (2, 3, 37, 12), "normal", (0.5, 0.9, 0.99, 1.0)),
    ("f32_one_vector", torch.float32, (1, 1, 1, 4), "normal", (0.25, 0.5, 1.0)),
    ("bf16_small", torch.bfloat16, (1, 2, 1, 8), "normal", (0.125, 0.5, 0.875)),
    ("bf16_t3", torch.bfloat16, (3, 5, 1000, 24), "t3", (0.999, 0.9999)),
    ("f32_multichunk", torch.float32, (1, 2, 8192, 64), "t3", (0.9999, 0.999)),
    ("bf16_multichunk", torch.bfloat16, (4, 3, 4096, 40), "normal", (0.9999, 0.99)),
]


@pytest.mark.parametrize("name,dtype,shape,law,ratios", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_random(fa, name, dtype, shape, law, ratios):
    sigma = synth.head_sigmas(shape[1], seed=sum(name.encode()) % 1000)
    x = synth.activations(shape, sigma, law=law, outlier_frac=0.0005, outlier_mult=40.0, dtype=dtype,
                          seed=7 + len(name))
    _check(fa, x, ratios, name)


def test_coarse_values_heavy_ties(fa):
    rng = np.random.default_rng(5)
    B, H, S, D = 2, 4, 700, 32
    vals = (rng.integers(-24, 25, size=(B, H, S, D)) * 0.25).astype(np.float32)
    vals[:, 1] = np.round(vals[:, 1] / 4)  # even coarser head
    x = torch.from_numpy(vals).to(torch.bfloat16)
    _check(fa, x, (0.9, 0.99, 0.999, 0.9999, 1.0), "coarse")
    _check(fa, x.to(torch.float32), (0.99, 0.999), "coarse_f32")


def test_special_heads(fa):
    B, H, S, D = 2, 6, 256, 16
    n_per_b = S * D
    x = np.zeros((B, H, S, D), np.float32)
    x[:, 0] = -1.5                                                  # constant head
    zeros = np.where(np.arange(B * n_per_b) % 3 == 0, -0.0, 0.0).astype(np.float32)
    zeros[::7] = 1e-3
    x[:, 1] = zeros.reshape(B, S, D)                                # signed zeros
    ramp = np.arange(B * n_per_b, dtype=np.float32) * np.float32(0.5)
    x[:, 2] = ramp.reshape(B, S, D)                                 # ascending in memory order
    x[:, 3] = ramp[::-1].reshape(B, S, D)                           # descending in memory order
    x[:, 4] = 0.0                                                   # all +0 (scale 0 later)
    x[:, 5] = -ramp[::-1].reshape(B, S, D)                          # negative descending
    xt = torch.from_numpy(x)
    _check(fa, xt, (0.9, 0.999, 1.0), "special_f32")
    _check(fa, xt.to(torch.bfloat16), (0.5, 0.99, 0.9999), "special_bf16")


def test_k4196_long_context_shape(fa):
    # bf16 (2,2,16384,128) with t3 tails and 1e-4 outliers at +-60 sigma; ratio 0.999 -> K = 4196
    sigma = synth.head_sigmas(2, seed=55)
    x = synth.activations((2, 2, 16384, 128), sigma, law="t3", outlier_frac=1e-4, outlier_mult=60.0,
                          dtype=torch.bfloat16, seed=56)
    _check(fa, x, (0.999, 0.99999), "k4196")


def test_k4196_on_the_tail_lists(fa):
    # K = 4196 on heads of 786,432 values (below 2^20: the tail lists, estimated bound and
    # side merge), the long-context window count
    B, H, S, D = 2, 2, 4096, 96
    N = B * S * D
    ratio = (N - 4196 + 1 + 0.5) / N
    assert N - int(ratio * N) + 1 == 4196
    sigma = synth.head_sigmas(H, seed=61)
    x = synth.activations((B, H, S, D), sigma, law="t3", outlier_frac=1e-4, outlier_mult=60.0,
                          dtype=torch.bfloat16, seed=62)
    _check(fa, x, (ratio,), "k4196_tail")


def test_batches_accumulate_and_scale(fa):
    dev = torch.device("cuda:0")
    H = 6
    sigma = synth.head_sigmas(H, seed=61)
    run_min = torch.empty(H, dtype=torch.float32, device=dev)
    run_max = torch.empty(H, dtype=torch.float32, device=dev)
    fa.fa3q_init_minmax(run_min, run_max)
    omin, omax = oracle.init_running(H)
    for bidx in range(4):
        x = synth.activations((2, H, 512, 32), sigma, law="t3", dtype=torch.bfloat16, seed=70 + bidx)
        log(f"accumulate batch {bidx}")
        wmin, wmax = fa.fa3q_calibrate_perhead(x.to(dev), 0.999)
        fa.fa3q_accumulate_minmax(run_min, run_max, wmin, wmax)
        cmin, cmax = oracle.calibrate(_host_f32(x), 0.999)
        omin, omax = oracle.accumulate(omin, omax, cmin, cmax)
    scale = fa.fa3q_qparams(run_min, run_max)
    torch.cuda.synchronize()
    assert_bits_equal(f32(run_min), omin, "run_min")
    assert_bits_equal(f32(run_max), omax, "run_max")
    assert_bits_equal(f32(scale), oracle.qparams(omin, omax), "scale")


def test_accumulate_signed_zero_and_identity(fa):
    dev = torch.device("cuda:0")
    a = torch.tensor([0.0, -0.0, 1.0, -2.0], device=dev)
    b = torch.tensor([-0.0, 0.0, -1.0, 5.0], device=dev)
    run_min = a.clone()
    run_max = b.clone()
    fa.fa3q_accumulate_minmax(run_min, run_max, b, a)
    torch.cuda.synchronize()
    omin, omax = oracle.accumulate(a.cpu().numpy(), b.cpu().numpy(), b.cpu().numpy(), a.cpu().numpy())
    assert_bits_equal(f32(run_min), omin, "min")
    assert_bits_equal(f32(run_max), omax, "max")
    fa.fa3q_init_minmax(run_min, run_max)
    torch.cuda.synchronize()
    assert torch.isinf(run_min).all() and (run_min > 0).all()
    assert torch.isinf(run_max).all() and (run_max < 0).all()


def test_qparams_closed_form(fa):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(91)
    mn = (-np.abs(rng.standard_t(3, size=5000)) * np.exp(rng.uniform(-40, 40, size=5000))).astype(np.float32)
    mx = (np.abs(rng.standard_t(3, size=5000)) * np.exp(rng.uniform(-40, 40, size=5000))).astype(np.float32)
    mn[:4] = [0.0, -0.0, -127.0, -12.7]
    mx[:4] = [0.0, -0.0, 3.0, 1.0]
    s = fa.fa3q_qparams(torch.from_numpy(mn).to(dev), torch.from_numpy(mx).to(dev))
    torch.cuda.synchronize()
    assert_bits_equal(f32(s), oracle.qparams(mn, mx), "scale")


def test_large_k_uses_more_than_64k_lds(fa):
    # K ~ 1e4 (bf16) and K = 4097 (float32) need 100-150 KiB of LDS per workgroup
    rng = np.random.default_rng(17)
    x = torch.from_numpy((rng.standard_t(3, size=(2, 2, 4096, 64)) * 0.7).astype(np.float32))
    log(f"device LDS per block: {torch.cuda.get_device_properties(0)}")
    _check(fa, x.to(torch.bfloat16), (0.98,), "large_k_bf16")   # K = 10486
    _check(fa, x[:, :, :64], (0.5,), "large_k_f32")               # N = 8192, K = 4097


@pytest.mark.parametrize("dtype,S", [(torch.bfloat16, 4096), (torch.float32, 2048)], ids=["bf16", "f32"])
def test_largest_supported_window_count(fa, dtype, S):
    # K = fa3q_calibrate_max_windows(dtype) exactly: the chunk and merge buffers at their
    # largest (14950 bf16 windows, 7475 float32 ones, on 2 heads of S * 16 values)
    kmax = fa.fa3q_calibrate_max_windows(dtype)
    N = S * 16
    ratio = (N - kmax + 1 + 0.5) / N
    assert N - int(ratio * N) + 1 == kmax
    rng = np.random.default_rng(23)
    x = torch.from_numpy((rng.standard_t(3, size=(1, 2, S, 16)) * 0.9).astype(np.float32)).to(dtype)
    _check(fa, x, (ratio,), f"k_max_{kmax}")


def test_tails_across_many_binades(fa):
    # log-uniform magnitudes over 2^-60 .. 2^60: the K tail keys span more top bytes than
    # the counting sort takes, so the side merge sorts them bitonically; narrow tails (the
    # other cases) take the counting sort
    rng = np.random.default_rng(37)
    B, H, S, D = 1, 2, 8192, 112  # below 2^20 values per head: the tail lists
    mag = np.exp2(rng.uniform(-60.0, 60.0, size=(B, H, S, D)))
    x = (np.where(rng.random((B, H, S, D)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    _check(fa, xt, (0.99, 0.999), "wide_tails")


def test_more_chunk_lists_than_the_merge_prefix_holds(fa):
    # 2560 slabs of 128 values: one chunk per slab, so 2560 lists per head, past the
    # 2048-list prefix of the side merge, which then reads every list slot (unused ones
    # fail its filter); K = 329 on 327,680 values per head
    x = synth.activations((2560, 2, 16, 8), synth.head_sigmas(2, seed=51), law="t3", outlier_frac=0.001,
                          outlier_mult=40.0, dtype=torch.bfloat16, seed=52)
    _check(fa, x, (0.999,), "many_lists")


def _run_start(j: int, q_vecs: int) -> int:
    """First vector of sample run j: the library spreads 32 runs of 256 vectors over the
    head, run j inside [j * stride, (j + 1) * stride) at a fixed phase."""
    stride = max(256, q_vecs // 32)
    return j * stride + ((((((2 * j + 1) * 40503) & 0xFFFF) * (stride - 256)) >> 16) & ~7)


def _workspace_flags(fa, x: torch.Tensor, ratio: float) -> list:
    """The check flags (the workspace's last 256-byte block: low side of each head, then
    high side) after one call."""
    dev = torch.device("cuda:0")
    B, H, S, D = x.shape
    nbytes = fa.fa3q_calibrate_workspace_bytes(x.dtype, B, H, S, D, ratio)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    fa.fa3q_calibrate_perhead(x.to(dev), ratio, workspace=ws)
    torch.cuda.synchronize()
    return ws[nbytes - 256:nbytes - 256 + 8 * H].cpu().view(torch.int32).numpy().tolist()


def test_large_first_tokens_do_not_defeat_the_estimated_bound(fa):
    # every sequence starts with four tokens of large values (as attention-sink tokens
    # have): 4 slabs, so runs at multiples of 1/32 of the head would all start on a slab
    # start and sample every one of them; the run phases keep the sample representative,
    # the estimated bound holds and no head takes the fix-up pass
    B, H, S, D = 4, 2, 2048, 112  # below 2^20 values per head: the tail lists
    rng = np.random.default_rng(41)
    x = rng.standard_t(3, size=(B, H, S, D)).astype(np.float32)
    x[:, :, :4, :] = np.where(rng.random((B, H, 4, D)) < 0.5, -30.0, 30.0)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    _check(fa, xt, (0.999,), "first_tokens")
    assert _workspace_flags(fa, xt, 0.999) == [0] * (2 * H)


def test_estimated_bound_that_fails_is_redone_exactly(fa):
    # K = 9177 against 2048 sampled groups: the head bound is an estimate, checked by the
    # merge.  Values placed where the evenly spaced sample reads (runs of 256 vectors every
    # Q/32 vectors; a group is a thread's vectors of four consecutive runs) give every group
    # an extreme, so the sample bounds tightly while the head holds only 2048 values beyond
    # the bound: the check fails and the head is redone without a bound.  (Heads below 2^20
    # values: the tail lists.)
    B, H, S, D = 1, 2, 8192, 112
    vec = 8                                   # bf16 values per 16-byte vector
    q_vecs = B * S * D // vec                 # vectors per head
    rng = np.random.default_rng(23)
    x = np.ones((B, H, S * D), np.float32)
    x[0, 1] = rng.standard_normal(S * D).astype(np.float32)
    for g in range(8):
        lo_run, hi_run = _run_start(4 * g, q_vecs), _run_start(4 * g + 1, q_vecs)
        for t in range(256):
            x[0, 0, (lo_run + t) * vec] = -7.0        # head 0: both sides fail
            x[0, 0, (hi_run + t) * vec] = 9.0
            x[0, 1, (lo_run + t) * vec + 3] = -50.0   # head 1: the low side fails
    xt = torch.from_numpy(x.reshape(B, H, S, D)).to(torch.bfloat16)
    _check(fa, xt, (0.99,), "estimate_fails")
    _check(fa, xt, (0.999, 0.9999), "estimate_fails_other_ratios")
    # the check flags show which sides failed: both of head 0, the low side of head 1
    assert _workspace_flags(fa, xt, 0.99) == [1, 1, 1, 0]


BATCH_CASES = [
    # dtype, shape, ratio, batches: register merge; 16 batches; side merge (8 lists of K = 526); float32 keys
    (torch.bfloat16, (2, 4, 2048, 64), 0.999, 3),
    (torch.bfloat16, (2, 4, 2048, 64), 0.999, 16),
    (torch.bfloat16, (4, 3, 4096, 32), 0.999, 2),
    (torch.float32, (2, 4, 1024, 64), 0.999, 3),
]


@pytest.mark.parametrize("dtype,shape,ratio,nb", BATCH_CASES, ids=["bf16", "bf16_16", "bf16_side", "f32"])
def test_batches_in_one_call_match_the_oracle(fa, dtype, shape, ratio, nb):
    dev = torch.device("cuda:0")
    sigma = synth.head_sigmas(shape[1], seed=321)
    xs = [synth.activations(shape, sigma, law="t3", outlier_frac=0.0005, outlier_mult=40.0, dtype=dtype,
                            seed=330 + i) for i in range(nb)]
    log(f"calibrate_batches: {nb} x {shape} {dtype} ratio={ratio}")
    H = shape[1]
    rmin = torch.empty(H, dtype=torch.float32, device=dev)
    rmax = torch.empty(H, dtype=torch.float32, device=dev)
    wmin = torch.empty((nb, H), dtype=torch.float32, device=dev)
    wmax = torch.empty((nb, H), dtype=torch.float32, device=dev)
    fa.fa3q_calibrate_batches([x.to(dev) for x in xs], ratio, rmin, rmax, True, wmin, wmax)
    torch.cuda.synchronize()
    run_lo, run_hi = oracle.init_running(H)
    for i, x in enumerate(xs):
        olo, ohi = oracle.calibrate(_host_f32(x), ratio)
        assert_bits_equal(f32(wmin[i]), olo, f"batch {i} win_min")
        assert_bits_equal(f32(wmax[i]), ohi, f"batch {i} win_max")
        run_lo, run_hi = oracle.accumulate(run_lo, run_hi, olo, ohi)
    assert_bits_equal(f32(rmin), run_lo, "run_min")
    assert_bits_equal(f32(rmax), run_hi, "run_max")
    # init off: the running state carries over (a second call over the same batches changes nothing)
    fa.fa3q_calibrate_batches([x.to(dev) for x in xs[:2]], ratio, rmin, rmax, False)
    torch.cuda.synchronize()
    assert_bits_equal(f32(rmin), run_lo, "run_min carried")
    assert_bits_equal(f32(rmax), run_hi, "run_max carried")


def test_batches_equal_per_batch_calls_at_the_calibration_workload(fa):
    # 4 bf16 batches (8,128,2048,128), ratio 0.9999: one call against 4 calibrate + accumulate calls
    dev = torch.device("cuda:0")
    shape, ratio = (8, 128, 2048, 128), 0.9999
    sigma = synth.head_sigmas(128, seed=2024)
    xs = [synth.activations(shape, sigma, law="t3", dtype=torch.bfloat16, seed=100 + i, device=dev) for i in range(4)]
    log(f"calibrate_batches: 4 x {shape} ratio={ratio}")
    rmin = torch.empty(128, dtype=torch.float32, device=dev)
    rmax = torch.empty(128, dtype=torch.float32, device=dev)
    wmin = torch.empty((4, 128), dtype=torch.float32, device=dev)
    wmax = torch.empty((4, 128), dtype=torch.float32, device=dev)
    fa.fa3q_calibrate_batches(xs, ratio, rmin, rmax, True, wmin, wmax)
    qmin = torch.empty(128, dtype=torch.float32, device=dev)
    qmax = torch.empty(128, dtype=torch.float32, device=dev)
    fa.fa3q_init_minmax(qmin, qmax)
    for i, x in enumerate(xs):
        lo, hi = fa.fa3q_calibrate_perhead(x, ratio)
        torch.cuda.synchronize()
        assert torch.equal(lo.view(torch.int32), wmin[i].view(torch.int32)), i
        assert torch.equal(hi.view(torch.int32), wmax[i].view(torch.int32)), i
        fa.fa3q_accumulate_minmax(qmin, qmax, lo, hi)
    torch.cuda.synchronize()
    assert torch.equal(qmin.view(torch.int32), rmin.view(torch.int32))
    assert torch.equal(qmax.view(torch.int32), rmax.view(torch.int32))


def test_batches_with_an_estimated_bound_that_fails_in_one_batch(fa):
    # K = 9177 (estimated bounds): batch 1 plants the sampled-position extremes that make
    # its check fail; batches 0 and 2 are ordinary.  Each batch has its own flags and lists.
    # (Heads below 2^20 values: the tail lists.)
    dev = torch.device("cuda:0")
    B, H, S, D = 1, 2, 8192, 112
    vec, q_vecs = 8, B * S * D // 8
    rng = np.random.default_rng(29)
    xs = []
    for i in range(3):
        x = rng.standard_normal((B, H, S * D)).astype(np.float32)
        if i == 1:
            for g in range(8):
                for t in range(256):
                    x[0, :, (_run_start(4 * g, q_vecs) + t) * vec] = -70.0
                    x[0, :, (_run_start(4 * g + 1, q_vecs) + t) * vec] = 90.0
        xs.append(torch.from_numpy(x.reshape(B, H, S, D)).to(torch.bfloat16))
    rmin = torch.empty(H, dtype=torch.float32, device=dev)
    rmax = torch.empty(H, dtype=torch.float32, device=dev)
    wmin = torch.empty((3, H), dtype=torch.float32, device=dev)
    wmax = torch.empty((3, H), dtype=torch.float32, device=dev)
    log("calibrate_batches: estimated bound failing in batch 1")
    fa.fa3q_calibrate_batches([x.to(dev) for x in xs], 0.99, rmin, rmax, True, wmin, wmax)
    torch.cuda.synchronize()
    run_lo, run_hi = oracle.init_running(H)
    for i, x in enumerate(xs):
        olo, ohi = oracle.calibrate(_host_f32(x), 0.99)
        assert_bits_equal(f32(wmin[i]), olo, f"batch {i} win_min")
        assert_bits_equal(f32(wmax[i]), ohi, f"batch {i} win_max")
        run_lo, run_hi = oracle.accumulate(run_lo, run_hi, olo, ohi)
    assert_bits_equal(f32(rmin), run_lo, "run_min")
    assert_bits_equal(f32(rmax), run_hi, "run_max")
