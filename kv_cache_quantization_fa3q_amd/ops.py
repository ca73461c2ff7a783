"""torch-facing binding of libfa3q: same names as the C ABI, argument marshalling only.

Every function checks dtypes/devices/contiguity, allocates outputs and workspaces
with torch when the caller passes none, passes raw device pointers and the current
HIP stream to the library, and raises ``Fa3qError`` on a non-zero status.  All of
the path's arithmetic runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import FA3Q_BF16, FA3Q_F16, FA3Q_F32, Fa3qError, lib

__all__ = [
    "fa3q_calibrate_max_windows",
    "fa3q_calibrate_workspace_bytes",
    "fa3q_calibrate_perhead",
    "fa3q_calibrate_batches_workspace_bytes",
    "fa3q_calibrate_batches",
    "fa3q_init_minmax",
    "fa3q_accumulate_minmax",
    "fa3q_qparams",
    "fa3q_quantize_k",
    "fa3q_decode_attn_workspace_bytes",
    "fa3q_decode_attn",
    "fa3q_decode_attn_noalloc",
    "fa3q_decode_append_attn",
    "fa3q_decode_attn_qkv8",
    "fa3q_quantize_asym",
    "fa3q_decode_attn_asym",
    "fa3q_decode_latent_workspace_bytes",
    "fa3q_decode_latent",
    "dtype_code",
]


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return FA3Q_F32
    if dtype == torch.bfloat16:
        return FA3Q_BF16
    raise TypeError(f"unsupported dtype {dtype}; float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need_gpu(name: str, *tensors: Optional[torch.Tensor]) -> None:
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")


def _check(status: int, name: str) -> None:
    if status != 0:
        raise Fa3qError(status, name)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace


# --------------------------------------------------------------------------- calibration


def fa3q_calibrate_max_windows(dtype: torch.dtype) -> int:
    return int(lib().fa3q_calibrate_max_windows(dtype_code(dtype)))


def fa3q_calibrate_workspace_bytes(dtype: torch.dtype, B: int, H: int, S: int, D: int, ratio: float) -> int:
    return int(lib().fa3q_calibrate_workspace_bytes(dtype_code(dtype), B, H, S, D, float(ratio)))


def fa3q_calibrate_perhead(x: torch.Tensor, ratio: float, win_min: Optional[torch.Tensor] = None,
                           win_max: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Recall Window of every head of one batch ``x (B,H,S,D)`` -> ``(win_min[H], win_max[H])``."""
    if x.dim() != 4:
        raise ValueError("x must be (B, H, S, D)")
    B, H, S, D = (int(v) for v in x.shape)
    code = dtype_code(x.dtype)
    if win_min is None:
        win_min = torch.empty(H, dtype=torch.float32, device=x.device)
    if win_max is None:
        win_max = torch.empty(H, dtype=torch.float32, device=x.device)
    _need_gpu("fa3q_calibrate_perhead", x, win_min, win_max)
    nbytes = int(lib().fa3q_calibrate_workspace_bytes(code, B, H, S, D, float(ratio)))
    workspace = _workspace(nbytes, x.device, workspace)
    st = lib().fa3q_calibrate_perhead(_ptr(x), code, B, H, S, D, float(ratio), _ptr(win_min), _ptr(win_max),
                                      _ptr(workspace), nbytes if workspace is None else
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "fa3q_calibrate_perhead")
    return win_min, win_max


def fa3q_calibrate_batches_workspace_bytes(dtype: torch.dtype, nb: int, B: int, H: int, S: int, D: int,
                                           ratio: float) -> int:
    return int(lib().fa3q_calibrate_batches_workspace_bytes(dtype_code(dtype), nb, B, H, S, D, float(ratio)))


def fa3q_calibrate_batches(xs, ratio: float, run_min: torch.Tensor, run_max: torch.Tensor, init: bool = True,
                           win_min: Optional[torch.Tensor] = None, win_max: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Recall Windows of every batch in ``xs`` (same shape and dtype) folded into ``run_min``/``run_max``."""
    xs = list(xs)
    if not xs:
        raise ValueError("at least one batch")
    B, H, S, D = (int(v) for v in xs[0].shape)
    code = dtype_code(xs[0].dtype)
    for x in xs:
        if x.dim() != 4 or tuple(x.shape) != (B, H, S, D) or x.dtype != xs[0].dtype:
            raise ValueError("every batch must have the same (B, H, S, D) shape and dtype")
    _need_gpu("fa3q_calibrate_batches", *xs, run_min, run_max, win_min, win_max)
    nb = len(xs)
    nbytes = fa3q_calibrate_batches_workspace_bytes(xs[0].dtype, nb, B, H, S, D, ratio)
    workspace = _workspace(nbytes, xs[0].device, workspace)
    ptrs = (ctypes.c_void_p * nb)(*[x.data_ptr() for x in xs])
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_calibrate_batches(ptrs, nb, code, B, H, S, D, float(ratio), _ptr(run_min), _ptr(run_max),
                                      1 if init else 0, _ptr(win_min), _ptr(win_max), _ptr(workspace), wbytes,
                                      _stream(stream))
    _check(st, "fa3q_calibrate_batches")


def fa3q_init_minmax(run_min: torch.Tensor, run_max: torch.Tensor, stream=None) -> None:
    _need_gpu("fa3q_init_minmax", run_min, run_max)
    _check(lib().fa3q_init_minmax(_ptr(run_min), _ptr(run_max), run_min.numel(), _stream(stream)),
           "fa3q_init_minmax")


def fa3q_accumulate_minmax(run_min: torch.Tensor, run_max: torch.Tensor, cur_min: torch.Tensor,
                           cur_max: torch.Tensor, stream=None) -> None:
    _need_gpu("fa3q_accumulate_minmax", run_min, run_max, cur_min, cur_max)
    H = run_min.numel()
    if not (run_max.numel() == cur_min.numel() == cur_max.numel() == H):
        raise ValueError("all four statistics must have H elements")
    _check(lib().fa3q_accumulate_minmax(_ptr(run_min), _ptr(run_max), _ptr(cur_min), _ptr(cur_max), H,
                                        _stream(stream)), "fa3q_accumulate_minmax")


def fa3q_qparams(run_min: torch.Tensor, run_max: torch.Tensor, scale: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    H = run_min.numel()
    if scale is None:
        scale = torch.empty(H, dtype=torch.float32, device=run_min.device)
    _need_gpu("fa3q_qparams", run_min, run_max, scale)
    _check(lib().fa3q_qparams(_ptr(run_min), _ptr(run_max), _ptr(scale), H, _stream(stream)), "fa3q_qparams")
    return scale


# --------------------------------------------------------------------------- quantize


def fa3q_quantize_k(k: torch.Tensor, scale: torch.Tensor, Dn: int, k_nope_q: Optional[torch.Tensor] = None,
                    k_rope: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 ``k (B,H,S,Dn+Dr)`` -> ``(int8 k_nope_q (B,H,S,Dn), bf16 k_rope (B,H,S,Dr))``."""
    if k.dim() != 4 or k.dtype != torch.bfloat16:
        raise ValueError("k must be bfloat16 (B, H, S, Dn + Dr)")
    B, H, S, Dk = (int(v) for v in k.shape)
    Dr = Dk - int(Dn)
    if k_nope_q is None:
        k_nope_q = torch.empty((B, H, S, int(Dn)), dtype=torch.int8, device=k.device)
    if k_rope is None:
        k_rope = torch.empty((B, H, S, Dr), dtype=torch.bfloat16, device=k.device)
    _need_gpu("fa3q_quantize_k", k, scale, k_nope_q, k_rope)
    _check(lib().fa3q_quantize_k(_ptr(k), _ptr(scale), _ptr(k_nope_q), _ptr(k_rope) if Dr > 0 else None,
                                 B, H, S, int(Dn), Dr, _stream(stream)), "fa3q_quantize_k")
    return k_nope_q, k_rope


def fa3q_fake_quant(x: torch.Tensor, scale: torch.Tensor, Dn: int, y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """bf16 ``x (B,H,S,Dn+Dr)`` -> bf16 ``y``: the first Dn features quantised and dequantised
    per head, the rest copied.  ``y`` may be ``x`` itself (in place)."""
    if x.dim() != 4 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16 (B, H, S, Dn + Dr)")
    B, H, S, Dk = (int(v) for v in x.shape)
    if y is None:
        y = torch.empty_like(x)
    if y.shape != x.shape or y.dtype != torch.bfloat16:
        raise ValueError("y must be bfloat16 with x's shape")
    _need_gpu("fa3q_fake_quant", x, scale, y)
    _check(lib().fa3q_fake_quant(_ptr(x), _ptr(scale), _ptr(y), B, H, S, int(Dn), Dk - int(Dn), _stream(stream)),
           "fa3q_fake_quant")
    return y


# --------------------------------------------------------------------------- decode


def fa3q_decode_attn_workspace_bytes(B: int, H: int, T: int, Dv: int) -> int:
    return int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))


def fa3q_decode_attn(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, k_rope: torch.Tensor,
                     v: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Single-query attention over the INT8 K-nope + bf16 K-rope + bf16 V cache -> float32 ``(B,H,Dv)``."""
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError("k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    Dv = int(v.shape[-1])
    if q.shape != (B, H, Dn + Dr) or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dn + Dr)")
    if v.shape != (B, H, T, Dv) or v.dtype != torch.bfloat16:
        raise ValueError("v must be bfloat16 (B, H, T, Dv)")
    if k_rope is not None and (k_rope.shape != (B, H, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, H, T, Dr)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_attn", q, k_nope_q, scale, k_rope, v, out)
    nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
    workspace = _workspace(nbytes, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_attn(_ptr(q), _ptr(k_nope_q), _ptr(scale), _ptr(k_rope) if Dr > 0 else None, _ptr(v),
                                B, H, T, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace),
                                wbytes, _stream(stream))
    _check(st, "fa3q_decode_attn")
    return out


def fa3q_decode_attn_noalloc(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, k_rope: torch.Tensor,
                             v: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """``fa3q_decode_attn`` with no workspace: the library keeps the split states in its own static
    device array (``FA3Q_ERR_SCRATCH`` when they need more than it holds).  Calls that overlap in
    time on one GPU share that array and race; calls on one stream are ordered."""
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError("k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    Dv = int(v.shape[-1])
    if q.shape != (B, H, Dn + Dr) or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dn + Dr)")
    if v.shape != (B, H, T, Dv) or v.dtype != torch.bfloat16:
        raise ValueError("v must be bfloat16 (B, H, T, Dv)")
    if k_rope is not None and (k_rope.shape != (B, H, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, H, T, Dr)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_attn_noalloc", q, k_nope_q, scale, k_rope, v, out)
    st = lib().fa3q_decode_attn_noalloc(_ptr(q), _ptr(k_nope_q), _ptr(scale), _ptr(k_rope) if Dr > 0 else None,
                                        _ptr(v), B, H, T, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)), _ptr(out),
                                        _stream(stream))
    _check(st, "fa3q_decode_attn_noalloc")
    return out


def fa3q_decode_append_attn(q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                            scale: torch.Tensor, k_nope_q: torch.Tensor, k_rope: torch.Tensor, v: torch.Tensor,
                            kv_len: torch.Tensor, sm_scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step over a cache of capacity ``T``: with ``k_new``/``v_new`` the token is appended
    in place at position ``kv_len[b]`` and attention covers ``kv_len[b] + 1`` tokens; without them it
    covers ``kv_len[b]`` tokens.  Returns float32 ``(B,H,Dv)``; ``kv_len`` (int32 ``[B]``) is not changed."""
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError("k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    Dv = int(v.shape[-1])
    if q.shape != (B, H, Dn + Dr) or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dn + Dr)")
    if v.shape != (B, H, T, Dv) or v.dtype != torch.bfloat16:
        raise ValueError("v must be bfloat16 (B, H, T, Dv)")
    if k_rope is not None and (k_rope.shape != (B, H, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, H, T, Dr)")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new are given together or not at all")
    if k_new is not None:
        if k_new.shape != (B, H, Dn + Dr) or k_new.dtype != torch.bfloat16:
            raise ValueError("k_new must be bfloat16 (B, H, Dn + Dr)")
        if v_new.shape != (B, H, Dv) or v_new.dtype != torch.bfloat16:
            raise ValueError("v_new must be bfloat16 (B, H, Dv)")
    if kv_len.shape != (B,) or kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32 (B,)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_append_attn", q, k_new, v_new, scale, k_nope_q, k_rope, v, kv_len, out)
    nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
    workspace = _workspace(nbytes, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_append_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale), _ptr(k_nope_q),
                                       _ptr(k_rope) if Dr > 0 else None, _ptr(v), _ptr(kv_len), B, H, T, Dn, Dr,
                                       Dv, ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace), wbytes,
                                       _stream(stream))
    _check(st, "fa3q_decode_append_attn")
    return out


def fa3q_decode_paged_attn(q: torch.Tensor, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                           scale: torch.Tensor, k_nope_pool: torch.Tensor, k_rope_pool: Optional[torch.Tensor],
                           v_pool: torch.Tensor, block_table: torch.Tensor, kv_len: torch.Tensor, sm_scale: float,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """``fa3q_decode_append_attn`` over a paged cache: pools ``(num_pages, H, P, .)`` and an int32
    ``block_table (B, max_pages)`` of physical pages per logical page.  Returns float32 ``(B,H,Dv)``."""
    if k_nope_pool.dim() != 4 or k_nope_pool.dtype != torch.int8:
        raise ValueError("k_nope_pool must be int8 (num_pages, H, P, Dn)")
    NP, H, P, Dn = (int(s) for s in k_nope_pool.shape)
    Dr = int(k_rope_pool.shape[-1]) if k_rope_pool is not None else 0
    Dv = int(v_pool.shape[-1])
    if block_table.dim() != 2 or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 (B, max_pages)")
    B, MP = (int(s) for s in block_table.shape)
    if q.shape != (B, H, Dn + Dr) or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dn + Dr)")
    if v_pool.shape != (NP, H, P, Dv) or v_pool.dtype != torch.bfloat16:
        raise ValueError("v_pool must be bfloat16 (num_pages, H, P, Dv)")
    if k_rope_pool is not None and (k_rope_pool.shape != (NP, H, P, Dr) or k_rope_pool.dtype != torch.bfloat16):
        raise ValueError("k_rope_pool must be bfloat16 (num_pages, H, P, Dr)")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new are given together or not at all")
    if k_new is not None:
        if k_new.shape != (B, H, Dn + Dr) or k_new.dtype != torch.bfloat16:
            raise ValueError("k_new must be bfloat16 (B, H, Dn + Dr)")
        if v_new.shape != (B, H, Dv) or v_new.dtype != torch.bfloat16:
            raise ValueError("v_new must be bfloat16 (B, H, Dv)")
    if kv_len.shape != (B,) or kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32 (B,)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_paged_attn", q, k_new, v_new, scale, k_nope_pool, k_rope_pool, v_pool, block_table,
              kv_len, out)
    nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, MP * P, Dv))
    workspace = _workspace(nbytes, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_paged_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(scale), _ptr(k_nope_pool),
                                      _ptr(k_rope_pool) if Dr > 0 else None, _ptr(v_pool), _ptr(block_table),
                                      _ptr(kv_len), B, H, NP, P, MP, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)),
                                      _ptr(out), _ptr(workspace), wbytes, _stream(stream))
    _check(st, "fa3q_decode_paged_attn")
    return out


def fa3q_decode_attn_qkv8(q_nope_q: torch.Tensor, q_rope: Optional[torch.Tensor], scale_q: torch.Tensor,
                          k_nope_q: torch.Tensor, scale_k: torch.Tensor, k_rope: Optional[torch.Tensor],
                          v_q: torch.Tensor, scale_v: torch.Tensor, sm_scale: float,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Attention with INT8 query (non-RoPE part), K-nope and V, per-head scales -> float32 ``(B,H,Dv)``."""
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError("k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    if v_q.dim() != 4 or v_q.dtype != torch.int8 or tuple(v_q.shape[:3]) != (B, H, T):
        raise ValueError("v_q must be int8 (B, H, T, Dv)")
    Dv = int(v_q.shape[-1])
    if q_nope_q.shape != (B, H, Dn) or q_nope_q.dtype != torch.int8:
        raise ValueError("q_nope_q must be int8 (B, H, Dn)")
    if Dr > 0 and (q_rope is None or q_rope.shape != (B, H, Dr) or q_rope.dtype != torch.bfloat16):
        raise ValueError("q_rope must be bfloat16 (B, H, Dr)")
    if k_rope is not None and (k_rope.shape != (B, H, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, H, T, Dr)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=k_nope_q.device)
    _need_gpu("fa3q_decode_attn_qkv8", q_nope_q, q_rope if Dr > 0 else None, scale_q, k_nope_q, scale_k, k_rope,
              v_q, scale_v, out)
    nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
    workspace = _workspace(nbytes, k_nope_q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_attn_qkv8(_ptr(q_nope_q), _ptr(q_rope) if Dr > 0 else None, _ptr(scale_q),
                                     _ptr(k_nope_q), _ptr(scale_k), _ptr(k_rope) if Dr > 0 else None, _ptr(v_q),
                                     _ptr(scale_v), B, H, T, Dn, Dr, Dv, ctypes.c_float(float(sm_scale)), _ptr(out),
                                     _ptr(workspace), wbytes, _stream(stream))
    _check(st, "fa3q_decode_attn_qkv8")
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
    if k.dim() != 4 or k.dtype != torch.bfloat16:
        raise ValueError("k must be bfloat16 (B, H, S, Dn + Dr)")
    B, H, S, Dk = (int(v) for v in k.shape)
    Dr = Dk - int(Dn)
    code = _param_code("fa3q_quantize_asym", scale, offset, H, int(Dn))
    if k_nope_q is None:
        k_nope_q = torch.empty((B, H, S, int(Dn)), dtype=torch.int8, device=k.device)
    if k_rope is None:
        k_rope = torch.empty((B, H, S, Dr), dtype=torch.bfloat16, device=k.device)
    _need_gpu("fa3q_quantize_asym", k, scale, offset, k_nope_q, k_rope)
    _check(lib().fa3q_quantize_asym(_ptr(k), _ptr(scale), _ptr(offset), code, _ptr(k_nope_q),
                                    _ptr(k_rope) if Dr > 0 else None, B, H, S, int(Dn), Dr, _stream(stream)),
           "fa3q_quantize_asym")
    return k_nope_q, k_rope


def fa3q_decode_attn_asym(q: torch.Tensor, k_nope_q: torch.Tensor, scale: torch.Tensor, offset: torch.Tensor,
                          k_rope: Optional[torch.Tensor], v: torch.Tensor, sm_scale: float,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Single-query attention over the asymmetric INT8 K-nope cache -> float32 ``(B,H,Dv)``."""
    if k_nope_q.dim() != 4 or k_nope_q.dtype != torch.int8:
        raise ValueError("k_nope_q must be int8 (B, H, T, Dn)")
    B, H, T, Dn = (int(s) for s in k_nope_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    Dv = int(v.shape[-1])
    code = _param_code("fa3q_decode_attn_asym", scale, offset, H, Dn)
    if q.shape != (B, H, Dn + Dr) or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dn + Dr)")
    if v.shape != (B, H, T, Dv) or v.dtype != torch.bfloat16:
        raise ValueError("v must be bfloat16 (B, H, T, Dv)")
    if k_rope is not None and (k_rope.shape != (B, H, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, H, T, Dr)")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_attn_asym", q, k_nope_q, scale, offset, k_rope, v, out)
    nbytes = int(lib().fa3q_decode_attn_workspace_bytes(B, H, T, Dv))
    workspace = _workspace(nbytes, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_attn_asym(_ptr(q), _ptr(k_nope_q), _ptr(scale), _ptr(offset), code,
                                     _ptr(k_rope) if Dr > 0 else None, _ptr(v), B, H, T, Dn, Dr, Dv,
                                     ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace), wbytes,
                                     _stream(stream))
    _check(st, "fa3q_decode_attn_asym")
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
    if c_q.dim() == 4 and c_q.shape[1] == 1:
        c_q = c_q.view(c_q.shape[0], c_q.shape[2], c_q.shape[3])
    if k_rope is not None and k_rope.dim() == 4 and k_rope.shape[1] == 1:
        k_rope = k_rope.view(k_rope.shape[0], k_rope.shape[2], k_rope.shape[3])
    if c_q.dim() != 3 or c_q.dtype != torch.int8:
        raise ValueError("c_q must be int8 (B, T, Dl)")
    B, T, Dl = (int(v) for v in c_q.shape)
    Dr = int(k_rope.shape[-1]) if k_rope is not None else 0
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != Dl + Dr or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 (B, H, Dl + Dr)")
    H = int(q.shape[1])
    if k_rope is not None and (tuple(k_rope.shape) != (B, T, Dr) or k_rope.dtype != torch.bfloat16):
        raise ValueError("k_rope must be bfloat16 (B, T, Dr)")
    if scale.numel() != 1 or scale.dtype != torch.float32:
        raise ValueError("scale must be one float32 value")
    if out is None:
        out = torch.empty((B, H, Dl), dtype=torch.float32, device=q.device)
    _need_gpu("fa3q_decode_latent", q, c_q, scale, k_rope, out)
    nbytes = fa3q_decode_latent_workspace_bytes(B, H, T, Dl)
    workspace = _workspace(nbytes, q.device, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().fa3q_decode_latent(_ptr(q), _ptr(c_q), _ptr(scale), _ptr(k_rope) if Dr > 0 else None, B, H, T, Dl,
                                  Dr, ctypes.c_float(float(sm_scale)), _ptr(out), _ptr(workspace), wbytes,
                                  _stream(stream))
    _check(st, "fa3q_decode_latent")
    return out
