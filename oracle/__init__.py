"""fp64 CPU oracle for paged KV append + PagedAttention forward.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
"""
from .pa_oracle import (admitted, append_kv, derived_slot, effective_scale, explicit_slot, forward,
                        gather_sequence, locate_token, rope_key_fp16, rope_query_fp64,
                        token_position)

__all__ = ["admitted", "append_kv", "derived_slot", "effective_scale", "explicit_slot", "forward",
           "gather_sequence", "locate_token", "rope_key_fp16", "rope_query_fp64",
           "token_position"]
