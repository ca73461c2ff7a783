"""Tensor layouts of the per-head path (test infrastructure only).

The msModelSlim page "FA3量化" describes activations as ``(B, H, S, D)``; the MindIE pages'
KV cache for the decode phase gives no layout.  Reading L4: a tensor may also come as
``(B, S, H, D)`` (token-major, the layout of a projection's output before the heads are
split off); head ``h`` of row ``(b, s)`` is then ``x[b, s, h, :]``.  Every per-head quantity
(the head's multiset of values, its codes, its attention) is the one of the ``(B, H, S, D)``
tensor with axes 1 and 2 exchanged.
"""
from __future__ import annotations

import numpy as np

LAYOUTS = ("BHSD", "BSHD")


def to_bhsd(x, layout: str = "BHSD") -> np.ndarray:
    """View of a 4-D tensor in ``layout`` as ``(B, H, S, D)``."""
    x = np.asarray(x)
    if layout == "BHSD":
        return x
    if layout == "BSHD":
        return np.swapaxes(x, 1, 2)
    raise ValueError(f"unknown layout {layout!r}")


def from_bhsd(x, layout: str = "BHSD") -> np.ndarray:
    """A ``(B, H, S, D)`` tensor rearranged into ``layout`` (contiguous)."""
    return np.ascontiguousarray(to_bhsd(x, layout))
