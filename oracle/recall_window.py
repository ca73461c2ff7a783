"""Per-head calibration: Recall Window, cross-batch accumulation, symmetric scale.

Test infrastructure only (see the package header).  Follows the msModelSlim
page "FA3量化：Flash Attention 3激活量化算法说明", section 原理 -> 算法流程
(algorithm flow), whose steps are, in order:

1. per-head statistics: an activation ``x`` of shape ``(B, H, S, D)`` gives
   every head ``N = B*S*D`` data points of its own;
2. Recall Window on one head's ``head_data (N,)`` with ``ratio`` (0.9999 by
   default): sort, ``target_num = int(ratio*N)``, try every window start
   ``i = 0 .. N - target_num`` over the sorted data, window
   ``[sorted_data[i], sorted_data[i+target_num-1]]``, keep the shortest window,
   output its ``(min_val, max_val)``;
3. cross-batch accumulation: per batch a window, then running
   ``min_values[h] = min(...)`` and ``max_values[h] = max(...)``;
4. symmetric parameters: ``abs_max[h] = max(|min_values[h]|, |max_values[h]|)``
   and ``scale[h] = abs_max[h] / 127``.

Readings where the page is silent or ambiguous:

* R1 "reshape x to (H, N)": grouped per head (``x[:, h]`` flattened), since the
  page says each head collects its own N points; a raw row-major reshape of a
  ``(B,H,S,D)`` array would mix heads whenever ``B > 1``.
* R2 window starts run over ``0 .. N-target_num`` inclusive, i.e.
  ``N - target_num + 1`` windows ("all possible starts").
* R3 ``int(ratio*N)``: the product is an IEEE double and ``int`` truncates toward
  zero (Python semantics); ``ratio`` must lie in ``(0, 1]`` and the result must
  be at least 1, otherwise the call is rejected.
* R4 ties between equally short windows: the first (smallest start ``i``) wins.
* R5 ``window_length`` is a float32 subtraction (round to nearest even) of the
  float32 values of the two ends.
* R6 sort order: the float32 total order with ``-0.0 < +0.0``; non-finite input
  is rejected.
* R7 running min/max start at ``+inf`` / ``-inf`` and use the same total order.
* R8 ``abs_max / 127`` is one correctly rounded float32 division; a zero
  ``abs_max`` gives ``scale = 0``.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .floats import key_to_f32, total_order_key
from .layout import to_bhsd

DEFAULT_RATIO = 0.9999  # default ratio given for the Recall Window step


def per_head_view(x) -> np.ndarray:
    """``(B, H, S, D)`` -> ``(H, N)`` with ``N = B*S*D``, head by head (reading R1)."""
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("activation must be (B, H, S, D)")
    B, H, S, D = x.shape
    return np.transpose(x, (1, 0, 2, 3)).reshape(H, B * S * D)


def target_num(ratio: float, N: int) -> int:
    """``int(ratio * N)`` in double precision, truncated toward zero (reading R3)."""
    ratio = float(ratio)
    if not (0.0 < ratio <= 1.0):
        raise ValueError(f"ratio must be in (0, 1], got {ratio!r}")
    if N < 1:
        raise ValueError("a head needs at least one value")
    t = int(ratio * float(N))
    if t < 1:
        raise ValueError(f"int(ratio*N) = {t} < 1 (ratio={ratio!r}, N={N})")
    return t


def _sorted_total_order(values: np.ndarray) -> np.ndarray:
    """Ascending float32 values under the total order of reading R6."""
    return key_to_f32(np.sort(total_order_key(values)))


def recall_window(head_data, ratio: float = DEFAULT_RATIO) -> Tuple[np.float32, np.float32]:
    """Shortest window of sorted ``head_data`` holding ``target_num`` values.

    Returns ``(min_val, max_val)`` of that window as float32 scalars.
    """
    data = np.asarray(head_data, dtype=np.float32).reshape(-1)
    if not np.all(np.isfinite(data)):
        raise ValueError("head data must be finite")
    N = data.size
    sorted_data = _sorted_total_order(data)
    t = target_num(ratio, N)
    n_starts = N - t + 1  # i = 0 .. N - target_num, inclusive (reading R2)
    window_min = sorted_data[0:n_starts]
    window_max = sorted_data[t - 1:t - 1 + n_starts]
    with np.errstate(over="ignore"):
        window_length = window_max - window_min  # float32 RNE (reading R5)
    best = int(np.argmin(window_length))  # first occurrence of the minimum (R4)
    return window_min[best], window_max[best]


def calibrate(x, ratio: float = DEFAULT_RATIO, layout: str = "BHSD") -> Tuple[np.ndarray, np.ndarray]:
    """One calibration batch: the Recall Window of every head -> ``(min[H], max[H])``.

    ``x`` holds float32 values in ``layout`` (``"BHSD"``, or ``"BSHD"`` read as in
    ``oracle.layout``, reading L4)."""
    heads = per_head_view(to_bhsd(np.asarray(x, dtype=np.float32), layout))
    H = heads.shape[0]
    lo = np.empty(H, dtype=np.float32)
    hi = np.empty(H, dtype=np.float32)
    for h in range(H):
        lo[h], hi[h] = recall_window(heads[h], ratio)
    return lo, hi


def init_running(H: int) -> Tuple[np.ndarray, np.ndarray]:
    """Identity elements of the running statistics (reading R7)."""
    return np.full(H, np.inf, dtype=np.float32), np.full(H, -np.inf, dtype=np.float32)


def accumulate(min_values, max_values, current_min, current_max) -> Tuple[np.ndarray, np.ndarray]:
    """``min_values[h] = min(min_values[h], current_min[h])`` (and max), total order."""
    a = np.asarray(min_values, dtype=np.float32)
    b = np.asarray(current_min, dtype=np.float32)
    c = np.asarray(max_values, dtype=np.float32)
    d = np.asarray(current_max, dtype=np.float32)
    new_min = np.where(total_order_key(b) < total_order_key(a), b, a).astype(np.float32)
    new_max = np.where(total_order_key(d) > total_order_key(c), d, c).astype(np.float32)
    return new_min, new_max


def qparams(min_values, max_values) -> np.ndarray:
    """Symmetric per-head scale ``max(|min|, |max|) / 127`` in float32 (reading R8)."""
    mn = np.asarray(min_values, dtype=np.float32)
    mx = np.asarray(max_values, dtype=np.float32)
    abs_max = np.maximum(np.abs(mn), np.abs(mx)).astype(np.float32)
    return (abs_max / np.float32(127.0)).astype(np.float32)
