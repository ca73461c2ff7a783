"""CPU oracle for the FA3 per-head INT8 path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the GPU
library computes.  It exists to check the library, never to stand in for it:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code, constants or helpers with the
HIP library (``kv_cache_quantization_fa3q_amd``) and imports nothing from it.

Sources (the pages are cited by title and section):

* msModelSlim documentation page "FA3量化：Flash Attention 3激活量化算法说明"
  (FA3 quantization: Flash Attention 3 activation quantization algorithm),
  section 原理 -> 算法流程 (principle -> algorithm flow): the per-head view,
  the Recall Window search, cross-batch accumulation and the symmetric scale;
  section 适用要求 (requirements): INT8 symmetric only, parameters fixed after
  calibration.
* MindIE LLM user guide page "FA3 quantization", opening overview paragraph:
  only the non-RoPE part of K is quantised to 8 bits per head, the RoPE part of
  K stays in floating point, to shrink the KV cache for decode-phase attention.

Readings of points the pages leave open are listed in each module's header.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, closed forms, special cases, invariants or library
routines; none is "parity unpinned".
"""
from .floats import (bf16_bits_to_f32, bf16_bits_to_f64, bits16_to_f32, bits16_to_f64, f16_bits_to_f32, f16_bits_to_f64,
                     f32_to_bf16_bits_rne, key_to_f32, total_order_key)
from .layout import LAYOUTS, from_bhsd, to_bhsd
from .recall_window import (
    per_head_view,
    target_num,
    recall_window,
    calibrate,
    accumulate,
    init_running,
    qparams,
)
from .quant import quantize_k, dequantize_k_nope, fake_quant
from .attention import (attention_fp64, decode_attn, decode_append_attn, decode_paged_attn, decode_attn_qkv8,
                        decode_attn_asym, decode_attn_latent)
from .asym import params_to_f32, quantize_asym, dequantize_asym

__all__ = [
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "f16_bits_to_f32",
    "f16_bits_to_f64",
    "bits16_to_f32",
    "bits16_to_f64",
    "LAYOUTS",
    "to_bhsd",
    "from_bhsd",
    "f32_to_bf16_bits_rne",
    "total_order_key",
    "key_to_f32",
    "per_head_view",
    "target_num",
    "recall_window",
    "calibrate",
    "accumulate",
    "init_running",
    "qparams",
    "quantize_k",
    "dequantize_k_nope",
    "fake_quant",
    "attention_fp64",
    "decode_attn",
    "decode_append_attn",
    "decode_paged_attn",
    "decode_attn_qkv8",
    "decode_attn_latent",
    "decode_attn_asym",
    "params_to_f32",
    "quantize_asym",
    "dequantize_asym",
]
