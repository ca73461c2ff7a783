"""float16 input and (B,S,H,D) layouts on the GPU against the oracle.

Calibration (fa3q_calibrate_ex): bit-exact windows of every head, on the tail lists
(float16 (B,H,S,D) heads below 2^20 values) and on the histogram in all its shapes:
(B,H,S,D) slabs longer than a workgroup round, short rows stepped by the workgroup
((B,S,H,D) rows of D values, (B,H,S,D) slabs of a few tokens), rows that do not divide
the workgroup (idle lanes), one part or several per head, counters that wrap, and
running statistics over several batches.  Quantisation (fa3q_quantize_k_ex): every code
and RoPE value bit for bit, float16 and bf16, both layouts, zero and tiny scales.  Decode
(fa3q_decode_attn_ex, fa3q_decode_append_attn_ex): float16 and bf16 in both layouts within
the decode tolerances of the float64 oracle, the updated caches bit for bit, and the
(B,T,H,.) result identical to the (B,H,T,.) one on the same data.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DECODE_DESIGN_TOL, DECODE_TOL, assert_bits_equal, log, parallel, row_rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
NAMES = {torch.float16: "f16", torch.bfloat16: "bf16"}


@pytest.fixture(scope="module")
def fa():
    import kv_cache_quantization_fa3q_amd as m
    return m


def _bits(t: torch.Tensor) -> np.ndarray:
    """16-bit float tensor -> its uint16 patterns on the host."""
    assert t.dtype in NAMES
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _values(t: torch.Tensor) -> np.ndarray:
    """float32 values of a float32 / bf16 / float16 tensor, widened by the oracle."""
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy()
    return oracle.bits16_to_f32(_bits(t), NAMES[t.dtype])


def _bshd(t: torch.Tensor) -> torch.Tensor:
    return t.transpose(1, 2).contiguous()


def _oracle_windows(vals: np.ndarray, ratio: float, layout: str):
    heads = oracle.per_head_view(oracle.to_bhsd(vals, layout))
    res = parallel(lambda h: oracle.recall_window(heads[h], ratio), range(heads.shape[0]))
    return np.array([r[0] for r in res], np.float32), np.array([r[1] for r in res], np.float32)


def _activations(shape_bhsd, dtype, seed, layout):
    B, H, S, D = shape_bhsd
    sigma = synth.head_sigmas(H, seed=seed)
    x = synth.activations((B, H, S, D), sigma, law="t3", outlier_frac=0.0005, outlier_mult=20.0, dtype=dtype,
                          seed=seed + 1)
    return (x if layout == "BHSD" else _bshd(x)).to(DEV)


def _check_windows(fa, xs, ratio, layout, what):
    log(f"calibrate_ex {what}: nb={len(xs)} {xs[0].dtype} {layout} {tuple(xs[0].shape)} ratio={ratio}")
    wmin, wmax = fa.fa3q_calibrate_ex(xs, ratio, layout=layout)
    torch.cuda.synchronize()
    for b, x in enumerate(xs):
        lo, hi = _oracle_windows(_values(x), ratio, layout)
        assert_bits_equal(wmin[b].cpu().numpy(), lo, f"{what} batch {b} win_min")
        assert_bits_equal(wmax[b].cpu().numpy(), hi, f"{what} batch {b} win_max")


# ----------------------------------------------------------------------------- calibration

CASES = [
    # (what, dtype, layout, (B,H,S,D) in head-major order, ratios)
    ("f16 tail lists", torch.float16, "BHSD", (2, 4, 512, 64), (0.9999, 0.99, 0.9)),
    ("f16 histogram, 2 parts", torch.float16, "BHSD", (2, 8, 4096, 128), (0.999,)),
    ("bf16 BSHD rows, one part", torch.bfloat16, "BSHD", (2, 8, 2048, 128), (0.99, 0.5)),
    ("f16 BSHD rows, 4 parts", torch.float16, "BSHD", (2, 2, 8192, 128), (0.999,)),
    ("f16 BSHD rows of 24 vectors", torch.float16, "BSHD", (1, 4, 1000, 192), (0.9,)),
    ("bf16 BSHD rows of 1 vector", torch.bfloat16, "BSHD", (3, 5, 777, 8), (0.5, 0.99)),
    ("bf16 BHSD short slabs", torch.bfloat16, "BHSD", (512, 4, 16, 128), (0.999,)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_calibrate_ex_windows(fa, case):
    what, dtype, layout, shape, ratios = case
    x = _activations(shape, dtype, seed=900 + len(what), layout=layout)
    for ratio in ratios:
        _check_windows(fa, [x], ratio, layout, what)


def test_calibrate_ex_path_preconditions(fa):
    # the cases above reach the paths their names say (host-side plan facts)
    cap = fa.fa3q_calibrate_max_windows(torch.float16)
    B, H, S, D = CASES[0][3]
    N = B * S * D
    assert N < 1 << 20 and all(N - int(r * N) + 1 <= cap for r in CASES[0][4])
    assert CASES[1][3][0] * CASES[1][3][2] * CASES[1][3][3] >= 1 << 20
    assert (CASES[6][3][2] * CASES[6][3][3]) // 8 <= 1024 and math.prod(CASES[6][3]) // CASES[6][3][1] >= 1 << 20
    assert 1024 % (CASES[4][3][3] // 8) != 0


def test_calibrate_ex_degenerate_heads_bshd(fa):
    # per-pattern counts past 65535 in one part: constant and two-valued heads wrap the counters
    B, H, S, D = 2, 3, 1024, 64
    x = synth.activations((B, H, S, D), synth.head_sigmas(H, seed=950), dtype=torch.float16, seed=951)
    x[:, 0] = 1.5
    x[:, 1] = torch.where(torch.arange(S * D).reshape(S, D) % 2 == 0, 0.25, -0.25).to(torch.float16)
    x = _bshd(x).to(DEV)
    for ratio in (0.9, 0.5, 1.0):
        _check_windows(fa, [x], ratio, "BSHD", "degenerate heads")


def _many_distinct(shape_bhsd, seed, heavy=None):
    """float16 values spread log-uniformly over 16 binades of either sign: more distinct 16-bit
    patterns per head than the window search keeps as a list (so it takes the merge search);
    `heavy` = (head, count) repeats one value that many times in that head."""
    g = np.random.default_rng(seed)
    vals = np.exp2(g.uniform(-8.0, 8.0, size=shape_bhsd)) * np.where(g.random(shape_bhsd) < 0.5, -1.0, 1.0)
    x = torch.from_numpy(vals.astype(np.float16))
    if heavy is not None:
        h, count = heavy
        flat = x[:, h].reshape(-1)
        flat[g.choice(flat.numel(), size=count, replace=False)] = 0.75
        x[:, h] = flat.reshape(x[:, h].shape)
    return x


MANY = [
    # (what, layout, (B,H,S,D) head-major, heavy)
    ("one part", "BSHD", (2, 4, 2048, 128), None),
    ("two parts", "BHSD", (2, 4, 4096, 128), None),
    ("two parts, a value 100k times", "BHSD", (2, 4, 4096, 128), (1, 100000)),
    ("one part, a value 70k times", "BSHD", (2, 4, 2048, 128), (2, 70000)),
]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_calibrate_ex_many_distinct_f16(fa, case):
    what, layout, shape, heavy = case
    x = _many_distinct(shape, seed=940 + len(what), heavy=heavy)
    for h in range(shape[1]):
        assert len(np.unique(x[:, h].numpy().view(np.uint16))) > 24576  # past the list the search keeps
    x = (x if layout == "BHSD" else _bshd(x)).to(DEV)
    for ratio in (0.9999, 0.99, 0.5, 1.0):
        _check_windows(fa, [x], ratio, layout, f"many distinct, {what}")


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_calibrate_ex_running_statistics(fa, layout):
    B, H, S, D = 2, 4, 512, 64
    xs = [_activations((B, H, S, D), torch.float16, seed=960 + 7 * i, layout=layout) for i in range(3)]
    ratio = 0.999
    log(f"calibrate_ex running statistics: f16 {layout} nb=3 then nb=1")
    run_min = torch.empty(H, dtype=torch.float32, device=DEV)
    run_max = torch.empty(H, dtype=torch.float32, device=DEV)
    wmin = torch.empty((2, H), dtype=torch.float32, device=DEV)
    wmax = torch.empty((2, H), dtype=torch.float32, device=DEV)
    fa.fa3q_calibrate_ex(xs[:2], ratio, layout=layout, run_min=run_min, run_max=run_max, init=True, win_min=wmin,
                         win_max=wmax)
    fa.fa3q_calibrate_ex(xs[2:], ratio, layout=layout, run_min=run_min, run_max=run_max, init=False)
    scale = fa.fa3q_qparams(run_min, run_max)
    torch.cuda.synchronize()
    omin, omax = oracle.init_running(H)
    for b, x in enumerate(xs):
        lo, hi = _oracle_windows(_values(x), ratio, layout)
        if b < 2:
            assert_bits_equal(wmin[b].cpu().numpy(), lo, f"batch {b} win_min")
            assert_bits_equal(wmax[b].cpu().numpy(), hi, f"batch {b} win_max")
        omin, omax = oracle.accumulate(omin, omax, lo, hi)
    assert_bits_equal(run_min.cpu().numpy(), omin, "run_min")
    assert_bits_equal(run_max.cpu().numpy(), omax, "run_max")
    assert_bits_equal(scale.cpu().numpy(), oracle.qparams(omin, omax), "scale")


def test_calibrate_ex_equals_the_head_major_calls(fa):
    # float32 and bf16 (B,H,S,D) through the new entry point: the same windows as the batches call
    for dtype in (torch.float32, torch.bfloat16):
        x = _activations((2, 4, 256, 64), dtype, seed=970, layout="BHSD")
        log(f"calibrate_ex vs calibrate_batches: {dtype}")
        wmin, wmax = fa.fa3q_calibrate_ex([x, x], 0.99)
        rmin = torch.empty(4, dtype=torch.float32, device=DEV)
        rmax = torch.empty(4, dtype=torch.float32, device=DEV)
        bmin = torch.empty((2, 4), dtype=torch.float32, device=DEV)
        bmax = torch.empty((2, 4), dtype=torch.float32, device=DEV)
        fa.fa3q_calibrate_batches([x, x], 0.99, rmin, rmax, win_min=bmin, win_max=bmax)
        torch.cuda.synchronize()
        assert_bits_equal(wmin.cpu().numpy(), bmin.cpu().numpy(), "win_min")
        assert_bits_equal(wmax.cpu().numpy(), bmax.cpu().numpy(), "win_max")


# ----------------------------------------------------------------------------- quantisation

QCASES = [
    (torch.float16, "BHSD", 128, 64),
    (torch.float16, "BSHD", 128, 64),
    (torch.bfloat16, "BSHD", 128, 64),
    (torch.float16, "BSHD", 64, 32),
    (torch.float16, "BSHD", 48, 0),
]


@pytest.mark.parametrize("case", QCASES, ids=[f"{NAMES[c[0]]}-{c[1]}-{c[2]}+{c[3]}" for c in QCASES])
def test_quantize_k_ex_codes(fa, case):
    dtype, layout, Dn, Dr = case
    B, H, S = 2, 3, 300  # H below the 16 rows of an item: an item's rows wrap over the heads several times
    sigma = synth.head_sigmas(H, seed=980)
    k = synth.activations((B, H, S, Dn + Dr), sigma, law="t3", outlier_frac=0.001, outlier_mult=20.0, dtype=dtype,
                          seed=981)
    scale = (sigma.numpy().astype(np.float32) * np.float32(6.0) / np.float32(127.0)).astype(np.float32)
    scale[0] = np.float32(0.0)
    scale[2] = np.float32(1e-30)  # not a moderate normal scale: every code by the exact division
    kl = (k if layout == "BHSD" else _bshd(k)).to(DEV)
    log(f"quantize_k_ex {NAMES[dtype]} {layout} Dn={Dn} Dr={Dr}")
    codes, rope = fa.fa3q_quantize_k_ex(kl, torch.from_numpy(scale).to(DEV), Dn, layout=layout)
    torch.cuda.synchronize()
    oc, orope = oracle.quantize_k(_bits(kl), scale, Dn, dtype=NAMES[dtype], layout=layout)
    assert_bits_equal(codes.cpu().numpy(), oc, "codes")
    if Dr:
        assert rope.dtype == dtype
        assert_bits_equal(_bits(rope), orope, "rope")


def test_quantize_k_ex_bf16_head_major_equals_quantize_k(fa):
    B, H, S, Dn, Dr = 2, 4, 100, 128, 64
    sigma = synth.head_sigmas(H, seed=985)
    k = synth.activations((B, H, S, Dn + Dr), sigma, dtype=torch.bfloat16, seed=986).to(DEV)
    scale = torch.from_numpy((sigma.numpy() * 4.0 / 127.0).astype(np.float32)).to(DEV)
    log("quantize_k_ex bf16 BHSD vs quantize_k")
    c1, r1 = fa.fa3q_quantize_k_ex(k, scale, Dn)
    c2, r2 = fa.fa3q_quantize_k(k, scale, Dn)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(r1.view(torch.int16), r2.view(torch.int16))


# ----------------------------------------------------------------------------- decode


def _cache(B, H, T, Dn, Dr, Dv, dtype, seed):
    g = np.random.default_rng(seed)
    codes = g.integers(-127, 128, size=(B, H, T, Dn)).astype(np.int8)
    sigma = synth.head_sigmas(H, seed=seed)
    scale = (sigma.numpy().astype(np.float32) * np.float32(4.0) / np.float32(127.0)).astype(np.float32)
    rope = synth.activations((B, H, T, Dr), sigma, dtype=dtype, seed=seed + 1)
    v = synth.activations((B, H, T, Dv), sigma, dtype=dtype, seed=seed + 2)
    q = synth.normal_tensor((B, H, Dn + Dr), dtype=dtype, seed=seed + 3)
    return q, codes, scale, rope, v


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("T", [300, 9000])  # one split, several splits per (b, h)
def test_decode_attn_ex(fa, dtype, T):
    B, H, Dn, Dr, Dv = 2, 4, 128, 64, 128
    q, codes, scale, rope, v = _cache(B, H, T, Dn, Dr, Dv, dtype, seed=990 + T)
    sm = 1.0 / math.sqrt(Dn + Dr)
    outs = {}
    for layout in ("BHSD", "BSHD"):
        tr = (lambda t: t) if layout == "BHSD" else _bshd
        cq = tr(torch.from_numpy(codes)).to(DEV)
        log(f"decode_attn_ex {NAMES[dtype]} {layout} B={B} H={H} T={T}")
        outs[layout] = fa.fa3q_decode_attn_ex(q.to(DEV), cq, torch.from_numpy(scale).to(DEV), tr(rope).to(DEV),
                                              tr(v).to(DEV), sm, layout=layout)
    torch.cuda.synchronize()
    ref = oracle.decode_attn(_bits(q), codes, scale, _bits(rope), _bits(v), sm, dtype=NAMES[dtype])
    err = row_rel_err(outs["BHSD"].cpu().numpy(), ref)
    assert err <= DECODE_TOL and err <= DECODE_DESIGN_TOL, err
    # same data, same arithmetic in the same order: the layouts agree bit for bit
    assert_bits_equal(outs["BSHD"].cpu().numpy(), outs["BHSD"].cpu().numpy(), "BSHD vs BHSD")
    if dtype == torch.bfloat16:
        base = fa.fa3q_decode_attn(q.to(DEV), torch.from_numpy(codes).to(DEV), torch.from_numpy(scale).to(DEV),
                                   rope.to(DEV), v.to(DEV), sm)
        torch.cuda.synchronize()
        assert_bits_equal(outs["BHSD"].cpu().numpy(), base.cpu().numpy(), "decode_attn_ex vs decode_attn")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_decode_append_attn_ex(fa, dtype, layout):
    B, H, T, Dn, Dr, Dv = 3, 4, 5000, 128, 64, 128
    q, codes, scale, rope, v = _cache(B, H, T, Dn, Dr, Dv, dtype, seed=995)
    sigma = synth.head_sigmas(H, seed=995)
    k_new = synth.activations((B, H, 1, Dn + Dr), sigma, dtype=dtype, seed=996).reshape(B, H, Dn + Dr).contiguous()
    v_new = synth.activations((B, H, 1, Dv), sigma, dtype=dtype, seed=997).reshape(B, H, Dv).contiguous()
    kv_len = np.array([0, 2047, T - 1], np.int64)  # the first slot, one inside, the last slot
    sm = 1.0 / math.sqrt(Dn + Dr)
    tr = (lambda t: t) if layout == "BHSD" else _bshd
    cq = tr(torch.from_numpy(codes)).to(DEV)
    cr, cv = tr(rope).to(DEV), tr(v).to(DEV)
    log(f"decode_append_attn_ex {NAMES[dtype]} {layout} B={B} H={H} T={T} kv_len={list(kv_len)}")
    out = fa.fa3q_decode_append_attn_ex(q.to(DEV), k_new.to(DEV), v_new.to(DEV), torch.from_numpy(scale).to(DEV), cq,
                                        cr, cv, torch.tensor(kv_len, dtype=torch.int32, device=DEV), sm, layout=layout)
    torch.cuda.synchronize()
    name = NAMES[dtype]
    ref, rc, rr, rv = oracle.decode_append_attn(_bits(q), _bits(k_new), _bits(v_new), scale,
                                                codes if layout == "BHSD" else _bshd(torch.from_numpy(codes)).numpy(),
                                                _bits(tr(rope)), _bits(tr(v)), kv_len, sm, Dn, dtype=name,
                                                layout=layout)
    assert_bits_equal(cq.cpu().numpy(), rc, "codes after the append")
    assert_bits_equal(_bits(cr), rr, "rope after the append")
    assert_bits_equal(_bits(cv), rv, "v after the append")
    err = row_rel_err(out.cpu().numpy(), ref)
    assert err <= DECODE_TOL and err <= DECODE_DESIGN_TOL, err
