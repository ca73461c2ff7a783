"""Seeded synthetic inputs for the FA3 per-head INT8 path.

This module is shared by the CPU oracle checks, the GPU parity tests and the
benchmark.  It only draws random tensors of the workloads' shapes, value laws
and outlier structure; it contains none of the quantisation or attention
arithmetic, and it imports neither the oracle nor the HIP library.

Value laws (the pages give no data; these stand in for calibration activations
of a DeepSeek-style MLA layer, whose K-nope head is 128 wide with a 64-wide
RoPE part):

* ``sigma_h = exp(U(-1, 1))`` per head, so heads differ in range, which is the
  situation per-head quantisation is meant for (msModelSlim "FA3量化" page,
  section 简介 / background).
* ``normal``: ``x = sigma_h * z`` with ``z ~ N(0, 1)``.
* ``t3``: ``x = sigma_h * z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)``, a Student-t
  with 3 degrees of freedom (heavy tails).
* outliers: per head, ``max(1, round(frac * N_h))`` positions drawn uniformly
  with replacement over the head's ``N_h = B*S*D`` values, each set to
  ``+-mult * sigma_h`` with a fair-coin sign (a position drawn more than once
  keeps its last draw, so the bytes do not depend on the device's store order).
* the result is rounded once to the storage dtype (bf16 round-to-nearest-even
  via torch's cast, or kept in fp32).

All draws come from ``torch.Generator`` objects seeded explicitly, so a given
``(seed, device)`` always yields the same bytes.  Large tensors are produced
slab by slab to bound temporary memory.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

__all__ = [
    "head_sigmas",
    "activations",
    "normal_tensor",
    "bf16_bits",
    "from_bf16_bits",
]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def head_sigmas(H: int, seed: int) -> torch.Tensor:
    """Per-head scale ``exp(U(-1,1))`` as float32 on the CPU (same on every device)."""
    g = _gen(seed, "cpu")
    u = torch.rand(H, generator=g, dtype=torch.float64) * 2.0 - 1.0
    return torch.exp(u).to(torch.float32)


def _t3(shape, g, device) -> torch.Tensor:
    z0 = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi.add_(z * z)
    return z0 / torch.sqrt(chi / 3.0)


def activations(
    shape: Sequence[int],
    sigma: torch.Tensor,
    *,
    law: str = "normal",
    outlier_frac: float = 0.0,
    outlier_mult: float = 40.0,
    dtype: torch.dtype = torch.bfloat16,
    seed: int = 0,
    device="cpu",
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Draw a ``(B, H, S, D)`` activation tensor with per-head scale ``sigma[h]``.

    ``law`` is ``"normal"`` or ``"t3"``.  When ``outlier_frac > 0`` each head gets
    ``max(1, round(outlier_frac * B*S*D))`` outliers at ``+-outlier_mult*sigma[h]``.
    The draw is done one batch slab ``(H, S, D)`` at a time.
    """
    B, H, S, D = (int(v) for v in shape)
    dev = torch.device(device)
    g = _gen(seed, dev)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=dtype, device=dev)
    sig = sigma.to(device=dev, dtype=torch.float32).view(H, 1, 1)
    # Slab-wise draw keeps temporaries to one (H,S,D) float32 slab (times 5 for t3).
    for b in range(B):
        if law == "normal":
            z = torch.randn((H, S, D), generator=g, device=dev, dtype=torch.float32)
        elif law == "t3":
            z = _t3((H, S, D), g, dev)
        else:
            raise ValueError(f"unknown law {law!r}")
        out[b].copy_((z * sig).to(dtype))
        del z
    if outlier_frac > 0.0:
        n_h = B * S * D
        count = max(1, int(round(outlier_frac * n_h)))
        pos = torch.randint(0, n_h, (H, count), generator=g, device=dev, dtype=torch.int64)
        sign = torch.randint(0, 2, (H, count), generator=g, device=dev, dtype=torch.int64) * 2 - 1
        val = sign.to(torch.float32) * float(outlier_mult) * sig.view(H, 1)
        # head-view position p -> (b, rem) with rem inside the (S, D) slab of head h
        b_idx = pos // (S * D)
        rem = pos % (S * D)
        h_idx = torch.arange(H, device=dev, dtype=torch.int64).view(H, 1).expand(H, count)
        flat = (b_idx * H + h_idx) * (S * D) + rem
        # a position drawn more than once takes its last draw's value: an indexed store with
        # repeated indices leaves the winner unspecified on the GPU
        flat = flat.reshape(-1)
        uniq, inv = torch.unique(flat, return_inverse=True)
        draw = torch.arange(flat.numel(), device=dev, dtype=torch.int64)
        last = torch.full((uniq.numel(),), -1, device=dev, dtype=torch.int64)
        last.scatter_reduce_(0, inv, draw, reduce="amax")
        out.view(-1)[uniq] = val.reshape(-1)[last].to(dtype)
    return out


def normal_tensor(shape: Sequence[int], *, std: float = 1.0, dtype=torch.bfloat16,
                  seed: int = 0, device="cpu") -> torch.Tensor:
    """``N(0, std^2)`` tensor rounded once to ``dtype`` (used for decode queries)."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    z = torch.randn(tuple(int(v) for v in shape), generator=g, device=dev, dtype=torch.float32)
    return (z * float(std)).to(dtype)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Reinterpret a bfloat16 tensor as its raw 16-bit patterns (int16 view)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


def from_bf16_bits(bits: torch.Tensor) -> torch.Tensor:
    """Reinterpret raw 16-bit patterns (int16/uint16) as bfloat16."""
    if bits.dtype == torch.uint16:
        bits = bits.view(torch.int16)
    return bits.view(torch.bfloat16)


def outlier_count(frac: float, n_h: int) -> int:
    """Number of outlier draws per head for a head of ``n_h`` values."""
    return max(1, int(round(frac * n_h))) if frac > 0 else 0
