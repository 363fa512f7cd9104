"""ctypes declarations of the C ABI of libpa.so: the op (``include/pa.h``)
and the test and measurement entry points (``include/pa_testing.h``)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_DEVICE = 3

STAGES = {"append": 0, "decode": 1, "merge": 2, "prefill": 3, "plan": 4, "prefill_merge": 5,
          "q_norm": 6}

# entry points of include/pa.h, and of include/pa_testing.h
EXPORTED = ("pa_append_kv", "pa_forward_workspace_bytes", "pa_forward", "pa_forward_noalloc",
            "pa_last_error")
NOALLOC_SCRATCH_BYTES = 128 << 20     # PA_NOALLOC_SCRATCH_BYTES
TESTING_EXPORTED = ("pa_forward_workspace_bytes_routed", "pa_forward_routed", "pa_describe_plan",
                    "pa_timing_enable", "pa_timing_disable", "pa_timing_read",
                    "pa_bench_stream_read")


class AttnParams(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_num_heads", ctypes.c_int32),
                ("head_size", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
                ("local_window_size", ctypes.c_int32), ("do_rotary", ctypes.c_int32),
                ("rotary_interleaved", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
                ("k_quant_type", ctypes.c_int32), ("v_quant_type", ctypes.c_int32),
                ("head_sink", ctypes.c_void_p), ("use_smooth_softmax", ctypes.c_int32),
                ("q_norm_weight", ctypes.c_void_p), ("k_norm_weight", ctypes.c_void_p),
                ("qk_norm_epsilon", ctypes.c_float), ("kv_cache_layout", ctypes.c_int32),
                ("v_head_size", ctypes.c_int32), ("rotary_offset", ctypes.c_int32)]


class PagedKV(ctypes.Structure):
    _fields_ = [("key_cache", ctypes.c_void_p), ("value_cache", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("max_blocks_per_seq", ctypes.c_int32),
                ("cumulative_sequence_length", ctypes.c_void_p),
                ("past_seqlens", ctypes.c_void_p), ("batch_size", ctypes.c_int32),
                ("token_count", ctypes.c_int32), ("slot_mapping", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class Routing(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("prefill_pieces", ctypes.c_int32), ("prefill_kernel", ctypes.c_int32)]


_lib = None


class LibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libpa.so; raise loudly if it has not been built (there is no
    fallback implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_append_amd.build` "
            "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.pa_append_kv.argtypes = [P(AttnParams), P(PagedKV), vp, vp, vp, vp, i32, i32, vp]
    lib.pa_append_kv.restype = ctypes.c_int
    lib.pa_forward_workspace_bytes.argtypes = [P(AttnParams), P(PagedKV), i32, i32, P(sz)]
    lib.pa_forward_workspace_bytes.restype = ctypes.c_int
    lib.pa_forward.argtypes = [P(AttnParams), P(PagedKV), vp, vp, vp, i32, i32, i32, i32, vp,
                               sz, vp, vp]
    lib.pa_forward.restype = ctypes.c_int
    lib.pa_forward_noalloc.argtypes = [P(AttnParams), P(PagedKV), vp, vp, vp, i32, i32, i32, i32,
                                       vp, vp]
    lib.pa_forward_noalloc.restype = ctypes.c_int
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_forward_workspace_bytes_routed.argtypes = [P(AttnParams), P(PagedKV), P(Routing), i32,
                                                      i32, P(sz)]
    lib.pa_forward_workspace_bytes_routed.restype = ctypes.c_int
    lib.pa_forward_routed.argtypes = [P(AttnParams), P(PagedKV), P(Routing), vp, vp, vp, i32, i32,
                                      i32, i32, vp, sz, vp, vp]
    lib.pa_forward_routed.restype = ctypes.c_int
    lib.pa_describe_plan.argtypes = [P(AttnParams), P(PagedKV), P(Routing), i32, i32,
                                     ctypes.c_char_p, sz]
    lib.pa_describe_plan.restype = ctypes.c_int
    lib.pa_timing_enable.argtypes = [i32]
    lib.pa_timing_enable.restype = ctypes.c_int
    lib.pa_timing_disable.argtypes = []
    lib.pa_timing_disable.restype = ctypes.c_int
    lib.pa_timing_read.argtypes = [i32, P(ctypes.c_double), P(i32)]
    lib.pa_timing_read.restype = ctypes.c_int
    lib.pa_bench_stream_read.argtypes = [vp, sz, vp, vp]
    lib.pa_bench_stream_read.restype = ctypes.c_int
    _lib = lib
    return lib
