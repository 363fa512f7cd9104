"""fp64 CPU oracle for paged KV append + PagedAttention forward.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
"""
from .pa_oracle import (CACHE_FP8, CACHE_FP16, CACHE_INT8, LAYOUT_LATENT, LAYOUT_SEPARATE,
                        QK_NORM_EPSILON, QUANT_NONE,
                        QUANT_PER_CHANNEL, QUANT_PER_TENSOR, admitted, append_kv, dequantize, derived_slot,
                        effective_scale, explicit_slot, forward, fp8_e4m3fn_code, fp8_e4m3fn_codes,
                        fp8_e4m3fn_value, gather_codes, gather_sequence, locate_token, mapped_keys,
                        quantize_row, rms_norm_fp16, rope_key_fp16, rope_query_fp64,
                        token_position)

__all__ = ["CACHE_FP8", "CACHE_FP16", "CACHE_INT8", "LAYOUT_LATENT", "LAYOUT_SEPARATE",
           "QK_NORM_EPSILON", "QUANT_NONE", "QUANT_PER_CHANNEL",
           "QUANT_PER_TENSOR", "admitted", "append_kv", "dequantize", "derived_slot",
           "effective_scale", "explicit_slot", "forward", "fp8_e4m3fn_code", "fp8_e4m3fn_codes",
           "fp8_e4m3fn_value",
           "gather_codes", "gather_sequence", "locate_token", "mapped_keys", "quantize_row", "rms_norm_fp16", "rope_key_fp16",
           "rope_query_fp64", "token_position"]
