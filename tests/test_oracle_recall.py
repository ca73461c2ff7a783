"""Pins for the oracle's calibration stages (Recall Window, accumulation, scale).

Each check is independent of the oracle's own formulation: hand-worked cases
(tests/golden), two sort-free brute forces, closed forms, special cases and
invariants.  Source: msModelSlim page "FA3量化：Flash Attention 3激活量化算法说明",
section 原理 -> 算法流程.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "recall_window_cases.json")


def _bits(v):
    return int(np.asarray(v, dtype=np.float32).view(np.uint32))


def _tok(v):
    """Sortable integer for a float32 under the total order -0.0 < +0.0 (written independently)."""
    b = _bits(v)
    return -(b & 0x7FFFFFFF) - 1 if b >> 31 else b


def brute_by_lower_value(data, ratio):
    """Sort-free: for every distinct lower value a, the t-th smallest value >= a is the
    shortest upper end; keep the strictly shortest float32 length, scanning a upward."""
    vals = [np.float32(v) for v in data]
    t = int(ratio * len(vals))
    best = None
    for a in sorted(set(vals), key=_tok):
        above = sorted([v for v in vals if _tok(v) >= _tok(a)], key=_tok)
        if len(above) < t:
            continue
        b = above[t - 1]
        length = np.float32(b) - np.float32(a)
        if best is None or length < best[0]:
            best = (length, a, b)
    return best[1], best[2]


def brute_by_pairs(data, ratio):
    """Sort-free: every value interval [a, b] that covers >= t values; shortest float32
    length, then smallest a, then smallest b."""
    vals = np.asarray(data, dtype=np.float32)
    t = int(ratio * len(vals))
    toks = np.array([_tok(v) for v in vals])
    uniq = sorted(set(toks.tolist()))
    by_tok = {int(_tok(v)): np.float32(v) for v in vals}
    best = None
    for ta in uniq:
        for tb in uniq:
            if tb < ta:
                continue
            if int(np.sum((toks >= ta) & (toks <= tb))) < t:
                continue
            length = by_tok[tb] - by_tok[ta]
            key = (float(length), ta, tb)
            if best is None or key < best:
                best = key
    return by_tok[best[1]], by_tok[best[2]]


def _same(a, b):
    return _bits(a) == _bits(b)


# ----------------------------------------------------------------------------- golden


def test_golden_hand_worked_windows():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 5
    for c in cases:
        lo, hi = oracle.recall_window(np.array(c["data"], dtype=np.float32), c["ratio"])
        assert _same(lo, c["expected_min"]), c["name"]
        assert _same(hi, c["expected_max"]), c["name"]


def test_golden_scales():
    cases = json.load(open(GOLDEN))["scale_cases"]["cases"]
    for c in cases:
        s = oracle.qparams(np.array([c["min"]], np.float32), np.array([c["max"]], np.float32))[0]
        if "expected_scale" in c:
            assert _same(s, c["expected_scale"])
        else:
            absmax = max(abs(np.float32(c["min"])), abs(np.float32(c["max"])))
            assert _same(s, _round_f32(Fraction(float(absmax)) / 127))


# ----------------------------------------------------------------------------- brute force


@pytest.mark.parametrize("seed", range(60))
def test_matches_brute_force_with_duplicates(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 48))
    # coarse grid -> many ties and repeated values, both signs, signed zeros
    data = (rng.integers(-6, 7, size=n) * 0.5).astype(np.float32)
    if seed % 5 == 0:
        data[rng.integers(0, n)] = np.float32(-0.0)
    if seed % 7 == 0:
        data[rng.integers(0, n)] = np.float32(250.0)
    for ratio in (0.3, 0.5, 0.77, 0.9, 0.99, 1.0):
        if int(ratio * n) < 1:
            continue
        lo, hi = oracle.recall_window(data, ratio)
        blo, bhi = brute_by_lower_value(data, ratio)
        plo, phi = brute_by_pairs(data, ratio)
        assert _same(lo, blo) and _same(hi, bhi), (seed, ratio)
        assert _same(lo, plo) and _same(hi, phi), (seed, ratio)


@pytest.mark.parametrize("seed", range(20))
def test_matches_brute_force_continuous(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(20, 200))
    data = (rng.standard_t(3, size=n) * np.exp(rng.uniform(-1, 1))).astype(np.float32)
    for ratio in (0.5, 0.9, 0.97):
        lo, hi = oracle.recall_window(data, ratio)
        blo, bhi = brute_by_lower_value(data, ratio)
        assert _same(lo, blo) and _same(hi, bhi)


# ----------------------------------------------------------------------------- special cases


def test_ratio_one_gives_min_max():
    rng = np.random.default_rng(3)
    data = rng.normal(size=1000).astype(np.float32)
    lo, hi = oracle.recall_window(data, 1.0)
    assert lo == data.min() and hi == data.max()


def test_target_one_gives_smallest_value():
    data = np.array([4.0, -3.0, 2.0, 9.0, -3.0], np.float32)
    lo, hi = oracle.recall_window(data, 0.2)  # int(0.2*5) = 1
    assert lo == -3.0 and hi == -3.0


def test_arithmetic_progression_first_window():
    N = 257
    data = np.arange(N, dtype=np.float32)[::-1].copy()
    for ratio in (0.5, 0.9, 0.99):
        t = int(ratio * N)
        lo, hi = oracle.recall_window(data, ratio)
        assert lo == 0.0 and hi == float(t - 1)


def test_all_equal_head():
    data = np.full(333, -2.5, np.float32)
    lo, hi = oracle.recall_window(data, 0.9999)
    assert lo == -2.5 and hi == -2.5
    s = oracle.qparams(np.array([lo]), np.array([hi]))[0]
    assert _same(s, _round_f32(Fraction(2.5) / 127))


def test_far_outlier_excluded_when_two_windows():
    rng = np.random.default_rng(5)
    data = rng.normal(size=2048).astype(np.float32)
    data[77] = 1.0e6
    lo, hi = oracle.recall_window(data, 0.9999)  # target_num = 2047, two windows
    assert hi < 1.0e6 and lo == data.min()


def test_target_num_truncation_and_validation():
    assert oracle.target_num(0.9999, 2048) == 2047
    assert oracle.target_num(0.99, 2048) == 2027
    assert oracle.target_num(0.9999, 2097152) == 2096942
    assert oracle.target_num(0.999, 4194304) == 4190109
    assert oracle.target_num(0.99999, 4194304) == 4194262
    assert oracle.target_num(0.29, 100) == 28  # 0.29*100 = 28.999999999999996
    assert oracle.target_num(0.7, 10) == 7    # 0.7*10 = 7.0 exactly in double
    for bad in (0.0, -0.1, 1.0000001, float("nan")):
        with pytest.raises(ValueError):
            oracle.target_num(bad, 10)
    with pytest.raises(ValueError):
        oracle.target_num(0.05, 10)  # int(0.5) = 0 < 1


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        oracle.recall_window(np.array([1.0, np.inf], np.float32), 0.5)
    with pytest.raises(ValueError):
        oracle.recall_window(np.array([1.0, np.nan], np.float32), 0.5)


# ----------------------------------------------------------------------------- invariants


@pytest.mark.parametrize("seed", range(10))
def test_window_invariants(seed):
    rng = np.random.default_rng(77 + seed)
    n = int(rng.integers(100, 3000))
    data = (rng.standard_t(3, size=n)).astype(np.float32)
    prev_len = None
    for ratio in (0.5, 0.8, 0.9, 0.99, 0.999, 1.0):
        t = oracle.target_num(ratio, n)
        lo, hi = oracle.recall_window(data, ratio)
        assert np.sum((data >= lo) & (data <= hi)) >= t
        assert data.min() <= lo <= hi <= data.max()
        length = float(np.float32(hi) - np.float32(lo))
        # two-pointer over the sorted values: no run of t values is strictly shorter
        s = np.sort(data)
        runs = (s[t - 1:] - s[: n - t + 1]).astype(np.float32)
        assert length <= float(runs.min()) + 0.0
        if prev_len is not None:
            assert length >= prev_len  # a wider ratio never gives a shorter window
        prev_len = length


def test_per_head_grouping_does_not_mix_heads():
    # head 0 lives in [0,1), head 1 in [100,101); a raw reshape of (B,H,S,D) to (H,N)
    # with B=2 would put half of each head's values into the other row.
    rng = np.random.default_rng(9)
    B, H, S, D = 2, 2, 16, 8
    x = np.empty((B, H, S, D), np.float32)
    x[:, 0] = rng.uniform(0, 1, size=(B, S, D))
    x[:, 1] = rng.uniform(100, 101, size=(B, S, D))
    lo, hi = oracle.calibrate(x, 0.9)
    assert 0 <= lo[0] <= hi[0] < 1
    assert 100 <= lo[1] <= hi[1] < 101
    view = oracle.per_head_view(x)
    assert view.shape == (H, B * S * D)
    np.testing.assert_array_equal(np.sort(view[1]), np.sort(x[:, 1].reshape(-1)))


# ----------------------------------------------------------------------------- accumulate / qparams


def test_accumulate_identity_permutation_and_grouping():
    rng = np.random.default_rng(11)
    H = 16
    batches = [(rng.normal(size=H).astype(np.float32) - 2, rng.normal(size=H).astype(np.float32) + 2) for _ in range(5)]
    def run(order):
        mn, mx = oracle.init_running(H)
        for i in order:
            mn, mx = oracle.accumulate(mn, mx, *batches[i])
        return mn, mx
    a = run([0, 1, 2, 3, 4])
    b = run([4, 2, 0, 3, 1])
    np.testing.assert_array_equal(a[0], b[0]); np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[0], np.min([m for m, _ in batches], axis=0))
    np.testing.assert_array_equal(a[1], np.max([m for _, m in batches], axis=0))
    # first batch from the identity state is the batch itself
    mn, mx = oracle.init_running(H)
    mn, mx = oracle.accumulate(mn, mx, *batches[0])
    np.testing.assert_array_equal(mn, batches[0][0]); np.testing.assert_array_equal(mx, batches[0][1])


def test_accumulate_signed_zero_total_order():
    mn, mx = oracle.accumulate(np.array([0.0], np.float32), np.array([-0.0], np.float32),
                               np.array([-0.0], np.float32), np.array([0.0], np.float32))
    assert _bits(mn[0]) == 0x80000000 and _bits(mx[0]) == 0x00000000


def _round_f32(q: Fraction) -> np.float32:
    """Nearest float32 to a rational (ties to even mantissa), written independently."""
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    def dist(v):
        return abs(Fraction(float(v)) - q)
    best = min(cands, key=lambda v: (dist(v), int(np.asarray(v, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_qparams_correctly_rounded_division():
    rng = np.random.default_rng(13)
    mn = (-np.abs(rng.standard_t(3, size=4000)) * np.exp(rng.uniform(-30, 30, size=4000))).astype(np.float32)
    mx = (np.abs(rng.standard_t(3, size=4000)) * np.exp(rng.uniform(-30, 30, size=4000))).astype(np.float32)
    s = oracle.qparams(mn, mx)
    for i in range(len(s)):
        absmax = max(abs(float(mn[i])), abs(float(mx[i])))
        assert _same(s[i], _round_f32(Fraction(absmax) / 127)), i
        # 127*scale is within one float32 ulp of abs_max
        assert abs(float(np.float32(127) * s[i]) - absmax) <= float(np.spacing(np.float32(absmax)))
