"""torch-facing binding of libfa3q: same names as the C ABI, argument marshalling only.

Every function checks the dtype, shape, device and contiguity of every tensor it is
given (inputs, per-head statistics and caller-supplied outputs alike) and raises
``ValueError`` before anything is launched; it allocates the outputs and workspaces the
caller does not pass, passes raw device pointers to the library and raises ``Fa3qError``
on a non-zero status.  All of the path's arithmetic runs in the library's HIP kernels.

Streams: ``stream=None`` means torch's current stream; a ``torch.cuda.Stream`` or a raw
``hipStream_t`` handle (int) may be passed instead.  The wrapper then allocates its
outputs and workspaces while that stream is current, so torch's caching allocator ties
them to the stream the kernels run on (a workspace freed on return is reused only by
later work of that stream).  Inputs made on another stream must be ready before the
call, as for any torch op on a side stream.
"""
from __future__ import annotations

import contextlib
import ctypes
from typing import Iterator, Optional, Sequence, Tuple

import torch

from ._lib import FA3Q_BF16, FA3Q_BHSD, FA3Q_BSHD, FA3Q_F16, FA3Q_F32, Fa3qError, lib

__all__ = [
    "fa3q_calibrate_max_windows",
    "fa3q_calibrate_workspace_bytes",
    "fa3q_calibrate_perhead",
    "fa3q_calibrate_batches_workspace_bytes",
    "fa3q_calibrate_batches",
    "fa3q_calibrate_ex_workspace_bytes",
    "fa3q_calibrate_ex",
    "fa3q_init_minmax",
    "fa3q_accumulate_minmax",
    "fa3q_qparams",
    "fa3q_quantize_k",
    "fa3q_quantize_k_ex",
    "fa3q_fake_quant",
    "fa3q_decode_attn_workspace_bytes",
    "fa3q_decode_attn",
    "fa3q_decode_attn_ex",
    "fa3q_decode_attn_noalloc",
    "fa3q_decode_append_attn",
    "fa3q_decode_append_attn_ex",
    "fa3q_decode_paged_attn",
    "fa3q_decode_attn_qkv8",
    "fa3q_quantize_asym",
    "fa3q_decode_attn_asym",
    "fa3q_decode_latent_workspace_bytes",
    "fa3q_decode_latent",
    "dtype_code",
    "layout_code",
]

_LAYOUTS = {"BHSD": FA3Q_BHSD, "BSHD": FA3Q_BSHD}


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return FA3Q_F32
    if dtype == torch.bfloat16:
        return FA3Q_BF16
    if dtype == torch.float16:
        return FA3Q_F16
    raise TypeError(f"unsupported dtype {dtype}; float32, bfloat16 or float16")


def layout_code(layout: str) -> int:
    try:
        return _LAYOUTS[layout]
    except KeyError:
        raise ValueError(f"unknown layout {layout!r}; 'BHSD' or 'BSHD'") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@contextlib.contextmanager
def _on_stream(stream, device) -> Iterator[ctypes.c_void_p]:
    """Makes the call's stream current for the wrapper's allocations; yields its handle."""
    if stream is None:
        s = torch.cuda.current_stream(device)
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        s = torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        yield ctypes.c_void_p(s.cuda_stream)


def _need_gpu(name: str, *tensors: Optional[torch.Tensor]) -> None:
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")


def _per_head(name: str, what: str, t: Optional[torch.Tensor], n: int) -> None:
    """Per-head statistics and scales: float32 with exactly n elements."""
    if t is None:
        raise ValueError(f"{name}: {what} is required")
    if t.dtype != torch.float32 or t.numel() != n:
        raise ValueError(f"{name}: {what} must be float32 with {n} elements, got {t.dtype} with {t.numel()}")


def _shaped(name: str, what: str, t: Optional[torch.Tensor], shape, dtype: torch.dtype) -> None:
    if t is None:
        raise ValueError(f"{name}: {what} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: {what} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _check(status: int, name: str) -> None:
    if status != 0:
        raise Fa3qError(status, name)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """The caller's workspace when it is large enough, else a new one (on the current stream)."""
    if nbytes == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _bhsd(shape, layout: str) -> Tuple[int, int, int, int]:
    """(B, H, S, D) of a 4-D tensor stored in `layout`."""
    layout_code(layout)
    if len(shape) != 4:
        raise ValueError(f"a 4-D {layout} tensor is required, got shape {tuple(shape)}")
    a, b, c, d = (int(v) for v in shape)
    return (a, b, c, d) if layout == "BHSD" else (a, c, b, d)


def _in_layout(B: int, H: int, S: int, last: int, layout: str) -> Tuple[int, int, int, int]:
    return (B, H, S, last) if layout == "BHSD" else (B, S, H, last)


# --------------------------------------------------------------------------- calibration


def fa3q_calibrate_max_windows(dtype: torch.dtype) -> int:
    return int(lib().fa3q_calibrate_max_windows(dtype_code(dtype)))


def fa3q_calibrate_workspace_bytes(dtype: torch.dtype, B: int, H: int, S: int, D: int, ratio: float) -> int:
    return int(lib().fa3q_calibrate_workspace_bytes(dtype_code(dtype), B, H, S, D, float(ratio)))


def fa3q_calibrate_perhead(x: torch.Tensor, ratio: float, win_min: Optional[torch.Tensor] = None,
                           win_max: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Recall Window of every head of one batch ``x (B,H,S,D)`` -> ``(win_min[H], win_max[H])``."""
    name = "fa3q_calibrate_perhead"
    B, H, S, D = _bhsd(x.shape, "BHSD")
    code = dtype_code(x.dtype)
    _need_gpu(name, x, win_min, win_max, workspace)
    for what, t in (("win_min", win_min), ("win_max", win_max)):
        if t is not None:
            _per_head(name, what, t, H)
    with _on_stream(stream, x.device) as hs:
        if win_min is None:
            win_min = torch.empty(H, dtype=torch.float32, device=x.device)
        if win_max is None:
            win_max = torch.empty(H, dtype=torch.float32, device=x.device)
        nbytes = int(lib().fa3q_calibrate_workspace_bytes(code, B, H, S, D, float(ratio)))
        workspace = _workspace(nbytes, x.device, workspace)
        st = lib().fa3q_calibrate_perhead(_ptr(x), code, B, H, S, D, float(ratio), _ptr(win_min), _ptr(win_max),
                                          _ptr(workspace), _nbytes(workspace), hs)
    _check(st, name)
    return win_min, win_max


def fa3q_calibrate_batches_workspace_bytes(dtype: torch.dtype, nb: int, B: int, H: int, S: int, D: int,
                                           ratio: float) -> int:
    return int(lib().fa3q_calibrate_batches_workspace_bytes(dtype_code(dtype), nb, B, H, S, D, float(ratio)))


def fa3q_calibrate_ex_workspace_bytes(dtype: torch.dtype, layout: str, nb: int, B: int, H: int, S: int, D: int,
                                      ratio: float) -> int:
    return int(lib().fa3q_calibrate_ex_workspace_bytes(dtype_code(dtype), layout_code(layout), nb, B, H, S, D,
                                                       float(ratio)))


def _calibrate(name: str, xs: Sequence[torch.Tensor], ratio: float, layout: str, run_min, run_max, init: bool,
               win_min, win_max, workspace, stream, ex: bool):
    xs = list(xs)
    if not xs:
        raise ValueError(f"{name}: at least one batch")
    B, H, S, D = _bhsd(xs[0].shape, layout)
    code = dtype_code(xs[0].dtype)
    for x in xs:
        if tuple(x.shape) != tuple(xs[0].shape) or x.dtype != xs[0].dtype:
            raise ValueError(f"{name}: every batch must have the same shape and dtype")
    nb = len(xs)
    if (run_min is None) != (run_max is None):
        raise ValueError(f"{name}: run_min and run_max are given together")
    if (win_min is None) != (win_max is None):
        raise ValueError(f"{name}: win_min and win_max are given together")
    for what, t in (("run_min", run_min), ("run_max", run_max)):
        if t is not None:
            _per_head(name, what, t, H)
    for what, t in (("win_min", win_min), ("win_max", win_max)):
        if t is not None:
            _per_head(name, what, t, nb * H)
    _need_gpu(name, *xs, run_min, run_max, win_min, win_max, workspace)
    lcode = layout_code(layout)
    with _on_stream(stream, xs[0].device) as hs:
        if run_min is None and win_min is None:  # windows only: they are the result
            win_min = torch.empty((nb, H), dtype=torch.float32, device=xs[0].device)
            win_max = torch.empty((nb, H), dtype=torch.float32, device=xs[0].device)
        nbytes = int(lib().fa3q_calibrate_ex_workspace_bytes(code, lcode, nb, B, H, S, D, float(ratio)))
        workspace = _workspace(nbytes, xs[0].device, workspace)
        ptrs = (ctypes.c_void_p * nb)(*[x.data_ptr() for x in xs])
        if ex:
            st = lib().fa3q_calibrate_ex(ptrs, nb, code, lcode, B, H, S, D, float(ratio), _ptr(run_min),
                                         _ptr(run_max), 1 if init else 0, _ptr(win_min), _ptr(win_max),
                                         _ptr(workspace), _nbytes(workspace), hs)
        else:
            st = lib().fa3q_calibrate_batches(ptrs, nb, code, B, H, S, D, float(ratio), _ptr(run_min), _ptr(run_max),
                                              1 if init else 0, _ptr(win_min), _ptr(win_max), _ptr(workspace),
                                              _nbytes(workspace), hs)
    _check(st, name)
    return win_min, win_max


def fa3q_calibrate_batches(xs, ratio: float, run_min: torch.Tensor, run_max: torch.Tensor, init: bool = True,
                           win_min: Optional[torch.Tensor] = None, win_max: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Recall Windows of every batch in ``xs`` (same (B,H,S,D) shape and dtype) folded into
    ``run_min``/``run_max``; the windows also go to ``win_min``/``win_max`` ``[nb][H]`` when given."""
    name = "fa3q_calibrate_batches"
    if run_min is None or run_max is None:
        raise ValueError(f"{name}: run_min and run_max are required")
    _calibrate(name, xs, ratio, "BHSD", run_min, run_max, init, win_min, win_max, workspace, stream, ex=False)


def fa3q_calibrate_ex(xs, ratio: float, layout: str = "BHSD", run_min: Optional[torch.Tensor] = None,
                      run_max: Optional[torch.Tensor] = None, init: bool = True,
                      win_min: Optional[torch.Tensor] = None, win_max: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """``fa3q_calibrate_batches`` for float32, bfloat16 or float16 batches in either layout
    (``(B,H,S,D)`` or ``(B,S,H,D)``).  With no running statistics the windows ``[nb][H]`` are
    returned (allocated when not given); otherwise ``(win_min, win_max)`` as passed."""
    return _calibrate("fa3q_calibrate_ex", xs, ratio, layout, run_min, run_max, init, win_min, win_max, workspace,
                      stream, ex=True)


def fa3q_init_minmax(run_min: torch.Tensor, run_max: torch.Tensor, stream=None) -> None:
    name = "fa3q_init_minmax"
    H = run_min.numel()
    _per_head(name, "run_min", run_min, H)
    _per_head(name, "run_max", run_max, H)
    _need_gpu(name, run_min, run_max)
    with _on_stream(stream, run_min.device) as hs:
        st = lib().fa3q_init_minmax(_ptr(run_min), _ptr(run_max), H, hs)
    _check(st, name)


def fa3q_accumulate_minmax(run_min: torch.Tensor, run_max: torch.Tensor, cur_min: torch.Tensor,
                           cur_max: torch.Tensor, stream=None) -> None:
    name = "fa3q_accumulate_minmax"
    H = run_min.numel()
    for what, t in (("run_min", run_min), ("run_max", run_max), ("cur_min", cur_min), ("cur_max", cur_max)):
        _per_head(name, what, t, H)
    _need_gpu(name, run_min, run_max, cur_min, cur_max)
    with _on_stream(stream, run_min.device) as hs:
        st = lib().fa3q_accumulate_minmax(_ptr(run_min), _ptr(run_max), _ptr(cur_min), _ptr(cur_max), H, hs)
    _check(st, name)


def fa3q_qparams(run_min: torch.Tensor, run_max: torch.Tensor, scale: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    name = "fa3q_qparams"
    H = run_min.numel()
    _per_head(name, "run_min", run_min, H)
    _per_head(name, "run_max", run_max, H)
    if scale is not None:
        _per_head(name, "scale", scale, H)
    _need_gpu(name, run_min, run_max, scale)
    with _on_stream(stream, run_min.device) as hs:
        if scale is None:
            scale = torch.empty(H, dtype=torch.float32, device=run_min.device)
        st = lib().fa3q_qparams(_ptr(run_min), _ptr(run_max), _ptr(scale), H, hs)
    _check(st, name)
    return scale


# --------------------------------------------------------------------------- quantize


def _quantize(name: str, k: torch.Tensor, scale: torch.Tensor, Dn: int, layout: str, k_nope_q, k_rope, stream,
              ex: bool):
    if k.dtype not in ((torch.bfloat16, torch.float16) if ex else (torch.bfloat16,)):
        raise ValueError(f"{name}: k must be {'bfloat16 or float16' if ex else 'bfloat16'}, got {k.dtype}")
    B, H, S, Dk = _bhsd(k.shape, layout)
    Dn = int(Dn)
    Dr = Dk - Dn
    if Dn <= 0 or Dr < 0:
        raise ValueError(f"{name}: need 0 < Dn <= {Dk}, got Dn = {Dn}")
    _per_head(name, "scale", scale, H)
    if k_nope_q is not None:
        _shaped(name, "k_nope_q", k_nope_q, _in_layout(B, H, S, Dn, layout), torch.int8)
    if k_rope is not None:
        _shaped(name, "k_rope", k_rope, _in_layout(B, H, S, Dr, layout), k.dtype)
    _need_gpu(name, k, scale, k_nope_q, k_rope)
    with _on_stream(stream, k.device) as hs:
        if k_nope_q is None:
            k_nope_q = torch.empty(_in_layout(B, H, S, Dn, layout), dtype=torch.int8, device=k.device)
        if k_rope is None:
            k_rope = torch.empty(_in_layout(B, H, S, Dr, layout), dtype=k.dtype, device=k.device)
        rope = _ptr(k_rope) if Dr > 0 else None
        if ex:
            st = lib().fa3q_quantize_k_ex(_ptr(k), _ptr(scale), _ptr(k_nope_q), rope, dtype_code(k.dtype),
                                          layout_code(layout), B, H, S, Dn, Dr, hs)
        else:
            st = lib().fa3q_quantize_k(_ptr(k), _ptr(scale), _ptr(k_nope_q), rope, B, H, S, Dn, Dr, hs)
    _check(st, name)
    return k_nope_q, k_rope


def fa3q_quantize_k(k: torch.Tensor, scale: torch.Tensor, Dn: int, k_nope_q: Optional[torch.Tensor] = None,
                    k_rope: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 ``k (B,H,S,Dn+Dr)`` -> ``(int8 k_nope_q (B,H,S,Dn), bf16 k_rope (B,H,S,Dr))``."""
    return _quantize("fa3q_quantize_k", k, scale, Dn, "BHSD", k_nope_q, k_rope, stream, ex=False)


def fa3q_quantize_k_ex(k: torch.Tensor, scale: torch.Tensor, Dn: int, layout: str = "BHSD",
                       k_nope_q: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``fa3q_quantize_k`` for bfloat16 or float16 ``k`` in either layout; the codes and the
    RoPE part (k's dtype) come back in k's layout."""
    return _quantize("fa3q_quantize_k_ex", k, scale, Dn, layout, k_nope_q, k_rope, stream, ex=True)


def fa3q_fake_quant(x: torch.Tensor, scale: torch.Tensor, Dn: int, y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """bf16 ``x (B,H,S,Dn+Dr)`` -> bf16 ``y``: the first Dn features quantised and dequantised
    per head, the rest copied.  ``y`` may be ``x`` itself (in place)."""
    name = "fa3q_fake_quant"
    if x.dim() != 4 or x.dtype != torch.bfloat16:
        raise ValueError(f"{name}: x must be bfloat16 (B, H, S, Dn + Dr)")
    B, H, S, Dk = (int(v) for v in x.shape)
    _per_head(name, "scale", scale, H)
    if y is not None:
        _shaped(name, "y", y, x.shape, torch.bfloat16)
    _need_gpu(name, x, scale, y)
    with _on_stream(stream, x.device) as hs:
        if y is None:
            y = torch.empty_like(x)
        st = lib().fa3q_fake_quant(_ptr(x), _ptr(scale), _ptr(y), B, H, S, int(Dn), Dk - int(Dn), hs)
    _check(st, name)
    return y


# --------------------------------------------------------------------------- decode


def fa3q_decode_attn_workspace_bytes(B: int, H: int, T: int, Dv: int) -> int:
    return int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))


def _cache_dims(name: str, k_nope_q: torch.Tensor, k_rope: Optional[torch.Tensor], v: torch.Tensor, layout: str,
                vdtype: torch.dtype) -> Tuple[int, int, int, int, int, int]:
    """(B, H, T, Dn, Dr, Dv) of an INT8 K-nope / K-rope / V cache, checked against each other."""
    if k_nope_q.dtype != torch.int8:
        raise ValueError(f"{name}: k_nope_q must be int8")
    B, H, T, Dn = _bhsd(k_nope_q.shape, layout)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    Dv = int(v.shape[-1])
    _shaped(name, "v", v, _in_layout(B, H, T, Dv, layout), vdtype)
    if k_rope is not None:
        _shaped(name, "k_rope", k_rope, _in_layout(B, H, T, Dr, layout), vdtype)
    return B, H, T, Dn, Dr, Dv


def _decode(name: str, q, k_nope_q, scale, k_rope, v, sm_scale, out, workspace, stream, layout: str, ex: bool,
            noalloc: bool = False):
    dt = q.dtype
    if dt not in ((torch.bfloat16, torch.float16) if ex else (torch.bfloat16,)):
        raise ValueError(f"{name}: q must be {'bfloat16 or float16' if ex else 'bfloat16'}, got {dt}")
    B, H, T, Dn, Dr, Dv = _cache_dims(name, k_nope_q, k_rope, v, layout, dt)
    _shaped(name, "q", q, (B, H, Dn + Dr), dt)
    _per_head(name, "scale", scale, H)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dv), torch.float32)
    _need_gpu(name, q, k_nope_q, scale, k_rope, v, out, workspace)
    with _on_stream(stream, q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
        rope = _ptr(k_rope) if Dr > 0 else None
        sm = ctypes.c_float(float(sm_scale))
        if noalloc:
            st = lib().fa3q_decode_attn_noalloc(_ptr(q), _ptr(k_nope_q), _ptr(scale), rope, _ptr(v), B, H, T, Dn, Dr,
                                                Dv, sm, _ptr(out), hs)
        else:
            nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
            workspace = _workspace(nbytes, q.device, workspace)
            if ex:
                st = lib().fa3q_decode_attn_ex(_ptr(q), _ptr(k_nope_q), _ptr(scale), rope, _ptr(v), dtype_code(dt),
                                               layout_code(layout), B, H, T, Dn, Dr, Dv, sm, _ptr(out),
                                               _ptr(workspace), _nbytes(workspace), hs)
            else:
                st = lib().fa3q_decode_attn(_ptr(q), _ptr(k_nope_q), _ptr(scale), rope, _ptr(v), B, H, T, Dn, Dr, Dv,
                                            sm, _ptr(out), _ptr(workspace), _nbytes(workspace), hs)
    _check(st, name)
    return out


def fa3q_decode_attn(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, k_rope: torch.Tensor,
                     v: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Single-query attention over the INT8 K-nope + bf16 K-rope + bf16 V cache -> float32 ``(B,H,Dv)``."""
    return _decode("fa3q_decode_attn", q, k_nope_q, scale, k_rope, v, sm_scale, out, workspace, stream, "BHSD",
                   ex=False)


def fa3q_decode_attn_ex(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, k_rope: Optional[torch.Tensor],
                        v: torch.Tensor, sm_scale: float, layout: str = "BHSD", out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``fa3q_decode_attn`` with bfloat16 or float16 ``q``/``k_rope``/``v`` and the cache in either
    layout (``(B,H,T,.)`` or ``(B,T,H,.)``)."""
    return _decode("fa3q_decode_attn_ex", q, k_nope_q, scale, k_rope, v, sm_scale, out, workspace, stream, layout,
                   ex=True)


def fa3q_decode_attn_noalloc(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, k_rope: torch.Tensor,
                             v: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """``fa3q_decode_attn`` with no workspace: the library keeps the split states in its own static
    device array (``FA3Q_ERR_SCRATCH`` when they need more than it holds).  Calls that overlap in
    time on one GPU share that array and race; calls on one stream are ordered."""
    return _decode("fa3q_decode_attn_noalloc", q, k_nope_q, scale, k_rope, v, sm_scale, out, None, stream, "BHSD",
                   ex=False, noalloc=True)


def _append(name: str, q, k_new, v_new, scale, k_nope_q, k_rope, v, kv_len, sm_scale, out, workspace, stream,
            layout: str, ex: bool):
    dt = q.dtype
    if dt not in ((torch.bfloat16, torch.float16) if ex else (torch.bfloat16,)):
        raise ValueError(f"{name}: q must be {'bfloat16 or float16' if ex else 'bfloat16'}, got {dt}")
    B, H, T, Dn, Dr, Dv = _cache_dims(name, k_nope_q, k_rope, v, layout, dt)
    _shaped(name, "q", q, (B, H, Dn + Dr), dt)
    _per_head(name, "scale", scale, H)
    if (k_new is None) != (v_new is None):
        raise ValueError(f"{name}: k_new and v_new are given together or not at all")
    if k_new is not None:
        _shaped(name, "k_new", k_new, (B, H, Dn + Dr), dt)
        _shaped(name, "v_new", v_new, (B, H, Dv), dt)
    _shaped(name, "kv_len", kv_len, (B,), torch.int32)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dv), torch.float32)
    _need_gpu(name, q, k_new, v_new, scale, k_nope_q, k_rope, v, kv_len, out, workspace)
    with _on_stream(stream, q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
        nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
        workspace = _workspace(nbytes, q.device, workspace)
        rope = _ptr(k_rope) if Dr > 0 else None
        sm = ctypes.c_float(float(sm_scale))
        if ex:
            st = lib().fa3q_decode_append_attn_ex(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale), _ptr(k_nope_q), rope,
                                                  _ptr(v), _ptr(kv_len), dtype_code(dt), layout_code(layout), B, H, T,
                                                  Dn, Dr, Dv, sm, _ptr(out), _ptr(workspace), _nbytes(workspace), hs)
        else:
            st = lib().fa3q_decode_append_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale), _ptr(k_nope_q), rope,
                                               _ptr(v), _ptr(kv_len), B, H, T, Dn, Dr, Dv, sm, _ptr(out),
                                               _ptr(workspace), _nbytes(workspace), hs)
    _check(st, name)
    return out


def fa3q_decode_append_attn(q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                            scale: torch.Tensor, k_nope_q: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                            kv_len: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step over a cache of capacity ``T``: with ``k_new``/``v_new`` the token is appended
    in place at position ``kv_len[b]`` and attention covers ``kv_len[b] + 1`` tokens; without them it
    covers ``kv_len[b]`` tokens.  Returns float32 ``(B,H,Dv)``; ``kv_len`` (int32 ``[B]``) is not changed."""
    return _append("fa3q_decode_append_attn", q, k_new, v_new, scale, k_nope_q, k_rope, v, kv_len, sm_scale, out,
                   workspace, stream, "BHSD", ex=False)


def fa3q_decode_append_attn_ex(q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                               scale: torch.Tensor, k_nope_q: torch.Tensor, k_rope: Optional[torch.Tensor],
                               v: torch.Tensor, kv_len: torch.Tensor, sm_scale: float, layout: str = "BHSD",
                               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """``fa3q_decode_append_attn`` with bfloat16 or float16 ``q``/``k_new``/``v_new``/cache values and
    the cache in either layout."""
    return _append("fa3q_decode_append_attn_ex", q, k_new, v_new, scale, k_nope_q, k_rope, v, kv_len, sm_scale, out,
                   workspace, stream, layout, ex=True)


def fa3q_decode_paged_attn(q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                           scale: torch.Tensor, k_nope_pool: torch.Tensor, k_rope_pool: Optional[torch.Tensor],
                           v_pool: torch.Tensor, block_table: torch.Tensor, kv_len: torch.Tensor, sm_scale: float,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """``fa3q_decode_append_attn`` over a paged cache: pools ``(num_pages, H, P, .)`` and an int32
    ``block_table (B, max_pages)`` of physical pages per logical page.  Returns float32 ``(B,H,Dv)``."""
    name = "fa3q_decode_paged_attn"
    if k_nope_pool.dim() != 4 or k_nope_pool.dtype != torch.int8:
        raise ValueError(f"{name}: k_nope_pool must be int8 (num_pages, H, P, Dn)")
    NP, H, P, Dn = (int(s) for s in k_nope_pool.shape)
    Dr = int(k_rope_pool.shape[-1]) if k_rope_pool is not None else 0
    Dv = int(v_pool.shape[-1])
    if block_table.dim() != 2 or block_table.dtype != torch.int32:
        raise ValueError(f"{name}: block_table must be int32 (B, max_pages)")
    B, MP = (int(s) for s in block_table.shape)
    _shaped(name, "q", q, (B, H, Dn + Dr), torch.bfloat16)
    _shaped(name, "v_pool", v_pool, (NP, H, P, Dv), torch.bfloat16)
    if k_rope_pool is not None:
        _shaped(name, "k_rope_pool", k_rope_pool, (NP, H, P, Dr), torch.bfloat16)
    _per_head(name, "scale", scale, H)
    if (k_new is None) != (v_new is None):
        raise ValueError(f"{name}: k_new and v_new are given together or not at all")
    if k_new is not None:
        _shaped(name, "k_new", k_new, (B, H, Dn + Dr), torch.bfloat16)
        _shaped(name, "v_new", v_new, (B, H, Dv), torch.bfloat16)
    _shaped(name, "kv_len", kv_len, (B,), torch.int32)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dv), torch.float32)
    _need_gpu(name, q, k_new, v_new, scale, k_nope_pool, k_rope_pool, v_pool, block_table, kv_len, out, workspace)
    with _on_stream(stream, q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
        nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, MP * P, Dv))
        workspace = _workspace(nbytes, q.device, workspace)
        st = lib().fa3q_decode_paged_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale), _ptr(k_nope_pool),
                                          _ptr(k_rope_pool) if Dr > 0 else None, _ptr(v_pool), _ptr(block_table),
                                          _ptr(kv_len), B, H, NP, P, MP, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)),
                                          _ptr(out), _ptr(workspace), _nbytes(workspace), hs)
    _check(st, name)
    return out


def fa3q_decode_attn_qkv8(q_nope_q: torch.Tensor, q_rope: Optional[torch.Tensor], scale_q: torch.Tensor,
                          k_nope_q: torch.Tensor, scale_k: torch.Tensor, k_rope: Optional[torch.Tensor],
                          v_q: torch.Tensor, scale_v: torch.Tensor, sm_scale: float,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Attention with INT8 query (non-RoPE part), K-nope and V, per-head scales -> float32 ``(B,H,Dv)``."""
    name = "fa3q_decode_attn_qkv8"
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError(f"{name}: k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    if v_q.dim() != 4 or v_q.dtype != torch.int8 or tuple(v_q.shape[:3]) != (B, H, T):
        raise ValueError(f"{name}: v_q must be int8 (B, H, T, Dv)")
    Dv = int(v_q.shape[-1])
    _shaped(name, "q_nope_q", q_nope_q, (B, H, Dn), torch.int8)
    if Dr > 0:
        _shaped(name, "q_rope", q_rope, (B, H, Dr), torch.bfloat16)
        _shaped(name, "k_rope", k_rope, (B, H, T, Dr), torch.bfloat16)
    for what, t in (("scale_q", scale_q), ("scale_k", scale_k), ("scale_v", scale_v)):
        _per_head(name, what, t, H)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dv), torch.float32)
    _need_gpu(name, q_nope_q, q_rope if Dr > 0 else None, scale_q, k_nope_q, scale_k, k_rope, v_q, scale_v, out,
              workspace)
    with _on_stream(stream, k_nope_q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dv), dtype=torch.float32, device=k_nope_q.device)
        nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
        workspace = _workspace(nbytes, k_nope_q.device, workspace)
        st = lib().fa3q_decode_attn_qkv8(_ptr(q_nope_q), _ptr(q_rope) if Dr > 0 else None, _ptr(scale_q),
                                         _ptr(k_nope_q), _ptr(scale_k), _ptr(k_rope) if Dr > 0 else None, _ptr(v_q),
                                         _ptr(scale_v), B, H, T, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)),
                                         _ptr(out), _ptr(workspace), _nbytes(workspace), hs)
    _check(st, name)
    return out


# --------------------------------------------------------------------------- asymmetric K cache


def _param_code(name: str, scale: torch.Tensor, offset: torch.Tensor, H: int, Dn: int) -> int:
    if scale.dtype != offset.dtype or scale.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"{name}: scale and offset must both be bfloat16 or both float16")
    if tuple(scale.shape) != (H, Dn) or tuple(offset.shape) != (H, Dn):
        raise ValueError(f"{name}: scale and offset must be (H, Dn) = ({H}, {Dn})")
    return FA3Q_BF16 if scale.dtype == torch.bfloat16 else FA3Q_F16


def fa3q_quantize_asym(k: torch.Tensor, scale: torch.Tensor, offset: torch.Tensor, Dn: int,
                       k_nope_q: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 ``k (B,H,S,Dn+Dr)`` and ``(H,Dn)`` scale / offset tables -> asymmetric int8 codes and bf16 RoPE part."""
    name = "fa3q_quantize_asym"
    if k.dim() != 4 or k.dtype != torch.bfloat16:
        raise ValueError(f"{name}: k must be bfloat16 (B, H, S, Dn + Dr)")
    B, H, S, Dk = (int(v) for v in k.shape)
    Dn = int(Dn)
    Dr = Dk - Dn
    code = _param_code(name, scale, offset, H, Dn)
    if k_nope_q is not None:
        _shaped(name, "k_nope_q", k_nope_q, (B, H, S, Dn), torch.int8)
    if k_rope is not None:
        _shaped(name, "k_rope", k_rope, (B, H, S, Dr), torch.bfloat16)
    _need_gpu(name, k, scale, offset, k_nope_q, k_rope)
    with _on_stream(stream, k.device) as hs:
        if k_nope_q is None:
            k_nope_q = torch.empty((B, H, S, Dn), dtype=torch.int8, device=k.device)
        if k_rope is None:
            k_rope = torch.empty((B, H, S, Dr), dtype=torch.bfloat16, device=k.device)
        st = lib().fa3q_quantize_asym(_ptr(k), _ptr(scale), _ptr(offset), code, _ptr(k_nope_q),
                                      _ptr(k_rope) if Dr > 0 else None, B, H, S, Dn, Dr, hs)
    _check(st, name)
    return k_nope_q, k_rope


def fa3q_decode_attn_asym(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, offset: torch.Tensor,
                          k_rope: Optional[torch.Tensor], v: torch.Tensor, sm_scale: float,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Single-query attention over the asymmetric INT8 K-nope cache -> float32 ``(B,H,Dv)``."""
    name = "fa3q_decode_attn_asym"
    B, H, T, Dn, Dr, Dv = _cache_dims(name, k_nope_q, k_rope, v, "BHSD", torch.bfloat16)
    code = _param_code(name, scale, offset, H, Dn)
    _shaped(name, "q", q, (B, H, Dn + Dr), torch.bfloat16)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dv), torch.float32)
    _need_gpu(name, q, k_nope_q, scale, offset, k_rope, v, out, workspace)
    with _on_stream(stream, q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
        nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
        workspace = _workspace(nbytes, q.device, workspace)
        st = lib().fa3q_decode_attn_asym(_ptr(q), _ptr(k_nope_q), _ptr(scale), _ptr(offset), code,
                                         _ptr(k_rope) if Dr > 0 else None, _ptr(v), B, H, T, Dn, Dr, Dv,
                                         ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace),
                                         _nbytes(workspace), hs)
    _check(st, name)
    return out


# --------------------------------------------------------------------------- shared-latent (absorbed MLA) cache


def fa3q_decode_latent_workspace_bytes(B: int, H: int, T: int, Dl: int) -> int:
    return int(lib().fa3q_decode_latent_workspace_bytes(B, H, T, Dl))


def fa3q_decode_latent(q: torch.Tensor, c_q: torch.Tensor, scale: torch.Tensor, k_rope: Optional[torch.Tensor],
                       sm_scale: float, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Attention of every head over one shared latent cache -> float32 ``(B,H,Dl)`` (latent space).

    ``q (B,H,Dl+Dr)`` bf16 absorbed query, ``c_q (B,T,Dl)`` int8 latent codes (or ``(B,1,T,Dl)``),
    ``scale`` float32 with one element, ``k_rope (B,T,Dr)`` bf16 (or ``(B,1,T,Dr)``) or None.
    """
    name = "fa3q_decode_latent"
    if c_q.dim() == 4 and c_q.shape[1] == 1:
        c_q = c_q.view(c_q.shape[0], c_q.shape[2], c_q.shape[3])
    if k_rope is not None and k_rope.dim() == 4 and k_rope.shape[1] == 1:
        k_rope = k_rope.view(k_rope.shape[0], k_rope.shape[2], k_rope.shape[3])
    if c_q.dim() != 3 or c_q.dtype != torch.int8:
        raise ValueError(f"{name}: c_q must be int8 (B, T, Dl)")
    B, T, Dl = (int(v) for v in c_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != Dl + Dr or q.dtype != torch.bfloat16:
        raise ValueError(f"{name}: q must be bfloat16 (B, H, Dl + Dr)")
    H = int(q.shape[1])
    if k_rope is not None:
        _shaped(name, "k_rope", k_rope, (B, T, Dr), torch.bfloat16)
    _per_head(name, "scale", scale, 1)
    if out is not None:
        _shaped(name, "out", out, (B, H, Dl), torch.float32)
    _need_gpu(name, q, c_q, scale, k_rope, out, workspace)
    with _on_stream(stream, q.device) as hs:
        if out is None:
            out = torch.empty((B, H, Dl), dtype=torch.float32, device=q.device)
        nbytes = fa3q_decode_latent_workspace_bytes(B, H, T, Dl)
        workspace = _workspace(nbytes, q.device, workspace)
        st = lib().fa3q_decode_latent(_ptr(q), _ptr(c_q), _ptr(scale), _ptr(k_rope) if Dr > 0 else None, B, H, T,
                                      Dl, Dr, ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace),
                                      _nbytes(workspace), hs)
    _check(st, name)
    return out
