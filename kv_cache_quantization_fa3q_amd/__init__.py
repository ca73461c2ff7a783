"""FA3 per-head INT8 KV quantisation for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa3q.so`` (hand-written HIP kernels behind the C ABI in
``include/fa3q.h``); this package only loads it and marshals torch tensors into
its calls.  Build the library with ``python -m kv_cache_quantization_fa3q_amd.build``.
"""
from ._lib import (  # noqa: F401
    FA3Q_BF16,
    FA3Q_BHSD,
    FA3Q_BSHD,
    FA3Q_F16,
    FA3Q_F32,
    FA3Q_OK,
    Fa3qError,
    SIGNATURES,
    lib,
    library_path,
    status_string,
)
from .ops import (  # noqa: F401
    dtype_code,
    layout_code,
    fa3q_accumulate_minmax,
    fa3q_calibrate_batches,
    fa3q_calibrate_batches_workspace_bytes,
    fa3q_calibrate_ex,
    fa3q_calibrate_ex_workspace_bytes,
    fa3q_calibrate_max_windows,
    fa3q_calibrate_perhead,
    fa3q_calibrate_workspace_bytes,
    fa3q_decode_append_attn,
    fa3q_decode_append_attn_ex,
    fa3q_decode_attn,
    fa3q_decode_attn_ex,
    fa3q_decode_attn_noalloc,
    fa3q_decode_attn_asym,
    fa3q_decode_attn_qkv8,
    fa3q_decode_attn_workspace_bytes,
    fa3q_decode_latent,
    fa3q_decode_latent_workspace_bytes,
    fa3q_decode_paged_attn,
    fa3q_fake_quant,
    fa3q_init_minmax,
    fa3q_qparams,
    fa3q_quantize_asym,
    fa3q_quantize_k,
    fa3q_quantize_k_ex,
)
