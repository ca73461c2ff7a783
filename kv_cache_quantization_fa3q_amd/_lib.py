"""ctypes loader for libfa3q.so with the C signatures of include/fa3q.h.

torch is imported before the library is opened: torch ships the HIP runtime
(``libamdhip64.so.7``) and the dynamic loader then resolves libfa3q's dependency
to that same, already loaded runtime, so torch's streams and device pointers are
valid inside the library.  There is no fallback: a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must be loaded before libfa3q, see module docstring)

LIB_NAME = "libfa3q.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

FA3Q_OK = 0
FA3Q_ERR_NULL = 1
FA3Q_ERR_DTYPE = 2
FA3Q_ERR_SHAPE = 3
FA3Q_ERR_RATIO = 4
FA3Q_ERR_ALIGN = 5
FA3Q_ERR_WORKSPACE = 6
FA3Q_ERR_HIP = 7
FA3Q_ERR_UNSUPPORTED = 8
FA3Q_ERR_ALIAS = 9
FA3Q_ERR_SCRATCH = 10
FA3Q_ERR_LAYOUT = 11

FA3Q_NOALLOC_SCRATCH_BYTES = 16 << 20  # include/fa3q.h

FA3Q_F32 = 0
FA3Q_BF16 = 1
FA3Q_F16 = 2

FA3Q_BHSD = 0
FA3Q_BSHD = 1

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fa3q.h exactly
SIGNATURES = {
    "fa3q_status_string": (ctypes.c_char_p, [_int]),
    "fa3q_version": (_int, []),
    "fa3q_calibrate_max_windows": (_i64, [_int]),
    "fa3q_calibrate_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _i64, ctypes.c_double]),
    "fa3q_calibrate_perhead": (_int, [_vp, _int, _i64, _i64, _i64, _i64, ctypes.c_double, _vp, _vp, _vp, _sz, _vp]),
    "fa3q_init_minmax": (_int, [_vp, _vp, _i64, _vp]),
    "fa3q_accumulate_minmax": (_int, [_vp, _vp, _vp, _vp, _i64, _vp]),
    "fa3q_qparams": (_int, [_vp, _vp, _vp, _i64, _vp]),
    "fa3q_quantize_k": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]),
    "fa3q_decode_attn_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa3q_decode_attn": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_float,
                                _vp, _vp, _sz, _vp]),
    "fa3q_decode_append_attn": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                       ctypes.c_float, _vp, _vp, _sz, _vp]),
    "fa3q_decode_attn_qkv8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                     ctypes.c_float, _vp, _vp, _sz, _vp]),
    "fa3q_quantize_asym": (_int, [_vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]),
    "fa3q_fake_quant": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp]),
    "fa3q_decode_paged_attn": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                      _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _sz, _vp]),
    "fa3q_decode_attn_asym": (_int, [_vp, _vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                     ctypes.c_float, _vp, _vp, _sz, _vp]),
    "fa3q_decode_latent_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa3q_calibrate_batches_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _i64, _i64, ctypes.c_double]),
    "fa3q_calibrate_batches": (_int, [ctypes.POINTER(_vp), _i64, _int, _i64, _i64, _i64, _i64, ctypes.c_double, _vp,
                                      _vp, _int, _vp, _vp, _vp, _sz, _vp]),
    "fa3q_decode_latent": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _sz,
                                  _vp]),
    "fa3q_decode_attn_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_float,
                                        _vp, _vp]),
    "fa3q_calibrate_ex_workspace_bytes": (_sz, [_int, _int, _i64, _i64, _i64, _i64, _i64, ctypes.c_double]),
    "fa3q_calibrate_ex": (_int, [ctypes.POINTER(_vp), _i64, _int, _int, _i64, _i64, _i64, _i64, ctypes.c_double, _vp,
                                 _vp, _int, _vp, _vp, _vp, _sz, _vp]),
    "fa3q_quantize_k_ex": (_int, [_vp, _vp, _vp, _vp, _int, _int, _i64, _i64, _i64, _i64, _i64, _vp]),
    "fa3q_decode_attn_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _i64, _i64, _i64, _i64, _i64, _i64,
                                   ctypes.c_float, _vp, _vp, _sz, _vp]),
    "fa3q_decode_append_attn_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _i64, _i64, _i64, _i64,
                                          _i64, _i64, ctypes.c_float, _vp, _vp, _sz, _vp]),
}

_lock = threading.Lock()
_lib = None


class Fa3qError(RuntimeError):
    """A libfa3q call returned a non-zero status."""

    def __init__(self, status: int, call: str):
        self.status = int(status)
        self.call = call
        super().__init__(f"{call} failed: {status_string(self.status)} (status {self.status})")


def lib() -> ctypes.CDLL:
    """The loaded library (opened on first use); raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m kv_cache_quantization_fa3q_amd.build` "
                    "(or __graft_entry__.build()); there is no non-HIP fallback")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fa3q_status_string(int(status)).decode()


def library_path() -> str:
    return LIB_PATH
