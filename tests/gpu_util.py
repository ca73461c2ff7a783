"""Helpers shared by the GPU parity tests (conversion of device tensors to the
oracle's NumPy representations and the comparison metrics)."""
import sys

import numpy as np
import torch

DECODE_TOL = 2e-2        # required bound: max row-normalised relative error vs the float64 oracle
DECODE_DESIGN_TOL = 1e-4  # tighter bound the float32-accumulating kernels are held to


def log(msg: str) -> None:
    """Name the case before a GPU step so a failing run says what it was doing."""
    print(msg, flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 patterns on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().astype(np.float32, copy=False)


def assert_bits_equal(a, b, what: str) -> None:
    """Bitwise equality of two float32 (or int) arrays, with the first mismatches named."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shapes {a.shape} vs {b.shape}"
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    diff = np.flatnonzero(a.reshape(-1) != b.reshape(-1))
    if len(diff):
        first = [(int(i), a.reshape(-1)[i].item(), b.reshape(-1)[i].item()) for i in diff[:5]]
        raise AssertionError(f"{what}: {len(diff)} of {a.size} differ; (flat index, gpu, oracle): {first}")


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (b, h) of max_j |out - ref| / max_j |ref|."""
    out = np.asarray(out, dtype=np.float64).reshape(-1, out.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    denom = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(out - ref).max(axis=1) / denom).max())


def host_threads() -> int:
    """Worker threads for oracle checks: the host cores this process may use (at most 16)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_windows(x: torch.Tensor, ratio: float, heads=None):
    """The oracle's Recall Window of every head (or of `heads`) of a (B,H,S,D) device tensor,
    computed head by head on a thread pool (numpy's sort runs outside the GIL).
    Returns float32 (lo[len], hi[len])."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    H = x.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    lo = np.empty(len(heads), np.float32)
    hi = np.empty(len(heads), np.float32)
    xh = x.detach().cpu()  # one copy to the host; heads are gathered there (exact widening to float32)

    def one(i):
        h = heads[i]
        lo[i], hi[i] = oracle.recall_window(xh[:, h].to(torch.float32).numpy().reshape(-1), ratio)

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        list(ex.map(one, range(len(heads))))
    return lo, hi


def parallel(fn, items):
    """fn over items on a thread pool of the host's cores (the oracle's numpy work runs outside
    the GIL); results in item order."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=host_threads()) as ex:
        return list(ex.map(fn, items))
