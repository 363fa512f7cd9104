"""MI355X-native paged KV append + PagedAttention forward (HIP, gfx950).

The compute lives in ``libpa.so`` (built from ``csrc/`` by ``build.py``)
behind the C ABI of ``include/pa.h``.  This module only marshals torch tensors
(device memory) and the current HIP stream into those calls; there is no
other implementation, and calling it without the built library raises.

Names mirror the C entry points: :func:`append_kv` (``pa_append_kv``),
:func:`forward` (``pa_forward``), :func:`forward_workspace_bytes`,
:func:`forward_noalloc` (``pa_forward_noalloc``), :func:`last_error`; and, from ``include/pa_testing.h``, :class:`Routing`
(``pa_routing``, taken by :func:`forward`, :func:`forward_workspace_bytes` and
:func:`describe_plan`), the ``timing_*`` helpers and :func:`stream_read`.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Any, Optional

from . import _lib

__all__ = ["PAError", "Attn", "Routing", "CACHE_FP16", "CACHE_INT8", "CACHE_FP8_E4M3FN", "LAYOUT_SEPARATE",
           "LAYOUT_LATENT", "QUANT_NONE", "forward_noalloc",
           "QUANT_PER_TENSOR", "QUANT_PER_CHANNEL", "append_kv", "forward", "forward_workspace_bytes",
           "describe_plan", "last_error", "timing_enable", "timing_disable", "timing_read",
           "stream_read", "library_path"]


# cache element types, scale granularities and cache layouts (the ABI enums of pa.h)
CACHE_FP16, CACHE_INT8, CACHE_FP8_E4M3FN = 0, 1, 2
LAYOUT_SEPARATE, LAYOUT_LATENT = 0, 1
QUANT_NONE, QUANT_PER_TENSOR, QUANT_PER_CHANNEL = 0, 1, 2


class PAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


@dataclass
class Attn:
    """Attributes of the op (``pa_attn_params``)."""
    num_heads: int
    kv_num_heads: int
    head_size: int
    block_size: int
    scale: float = 0.0
    softcap: float = 0.0
    local_window_size: int = -1
    do_rotary: int = 0
    rotary_interleaved: int = 0
    cache_dtype: int = CACHE_FP16
    k_quant_type: int = QUANT_NONE
    v_quant_type: int = QUANT_NONE
    head_sink: Any = None           # fp16 device tensor [num_heads] or None
    use_smooth_softmax: int = 0
    q_norm_weight: Any = None       # fp16 device tensors [head_size] or None (both or neither)
    k_norm_weight: Any = None
    qk_norm_epsilon: float = 0.0    # 0 -> 1e-6
    kv_cache_layout: int = LAYOUT_SEPARATE
    v_head_size: int = 0            # 0 -> head_size (LATENT: the V view of each row)
    rotary_offset: int = 0

    @property
    def out_head_size(self) -> int:
        """Channels per head of the output (v_head_size with a latent cache)."""
        if self.kv_cache_layout == LAYOUT_LATENT and self.v_head_size:
            return self.v_head_size
        return self.head_size

    def c(self) -> _lib.AttnParams:
        import torch
        _need(self.head_sink, "head_sink", torch.float16, (self.num_heads,))
        _need(self.q_norm_weight, "q_norm_weight", torch.float16, (self.head_size,))
        _need(self.k_norm_weight, "k_norm_weight", torch.float16, (self.head_size,))
        return _lib.AttnParams(self.num_heads, self.kv_num_heads, self.head_size,
                               self.block_size, float(self.scale), float(self.softcap),
                               self.local_window_size, self.do_rotary,
                               self.rotary_interleaved, self.cache_dtype,
                               self.k_quant_type, self.v_quant_type, _ptr(self.head_sink),
                               self.use_smooth_softmax, _ptr(self.q_norm_weight),
                               _ptr(self.k_norm_weight), float(self.qk_norm_epsilon),
                               self.kv_cache_layout, self.v_head_size, self.rotary_offset)


@dataclass
class Routing:
    """Forced kernel routing (``pa_routing`` of ``include/pa_testing.h``);
    all zeros is the automatic choice.  For tests: every choice computes the
    same function, only the rounding may differ."""
    path: int = 0
    split_tokens: int = 0
    prefill_pieces: int = 0
    prefill_kernel: int = 0

    def c(self) -> _lib.Routing:
        return _lib.Routing(self.path, self.split_tokens, self.prefill_pieces,
                            self.prefill_kernel)


def library_path() -> str:
    return _lib.LIB_PATH


def last_error() -> str:
    return _lib.load().pa_last_error().decode()


def _check(status: int):
    if status != _lib.PA_OK:
        raise PAError(status, last_error())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, shape=None):
    import torch
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _cache_dtypes(cache_dtype: int):
    import torch
    if cache_dtype == CACHE_INT8:
        return (torch.int8,)
    if cache_dtype == CACHE_FP8_E4M3FN:
        return (torch.uint8, torch.float8_e4m3fn)
    return (torch.float16,)


def _kv(attn: Attn, key_cache, value_cache, block_table, cum, past, token_count,
        slot_mapping=None, k_scale=None, v_scale=None) -> _lib.PagedKV:
    import torch
    dts = _cache_dtypes(attn.cache_dtype)
    if key_cache.dtype not in dts:
        raise ValueError(f"key_cache: expected dtype {dts[0]} for cache_dtype "
                         f"{attn.cache_dtype}, got {key_cache.dtype}")
    _need(key_cache, "key_cache", key_cache.dtype)
    _need(value_cache, "value_cache", key_cache.dtype, key_cache.shape)   # None when latent
    _need(block_table, "block_table", torch.int32)
    _need(cum, "cumulative_sequence_length", torch.int32, (block_table.shape[0] + 1,))
    _need(past, "past_seqlens", torch.int32, (block_table.shape[0],))
    if key_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("key_cache must be rank 4 and block_table rank 2")
    if slot_mapping is not None:
        _need(slot_mapping, "slot_mapping", torch.int32, (token_count,))
    _need(k_scale, "k_scale", torch.float32)
    _need(v_scale, "v_scale", torch.float32)
    return _lib.PagedKV(key_cache.data_ptr(), _ptr(value_cache), key_cache.shape[0],
                        block_table.data_ptr(), block_table.shape[1], cum.data_ptr(),
                        past.data_ptr(), block_table.shape[0], token_count,
                        _ptr(slot_mapping), _ptr(k_scale), _ptr(v_scale))


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rot(attn: Attn, cos_cache, sin_cache):
    import torch
    if cos_cache is None:
        return None, None, 0, 0
    _need(cos_cache, "cos_cache", torch.float16)
    _need(sin_cache, "sin_cache", torch.float16, cos_cache.shape)
    return cos_cache.data_ptr(), sin_cache.data_ptr(), cos_cache.shape[0], 2 * cos_cache.shape[1]


def append_kv(attn: Attn, key, value, key_cache, value_cache, block_table, cum, past,
              cos_cache=None, sin_cache=None, stream=None, slot_mapping=None, k_scale=None,
              v_scale=None) -> None:
    """``pa_append_kv``: scatter new K/V rows ``[T, Hkv*D]`` into the pools
    (in place); ``slot_mapping`` (int32 ``[T]``, -1 = no write) gives the
    write slots instead of the block table.  Quantized caches
    (``attn.cache_dtype``) take fp32 ``k_scale``/``v_scale`` (``[1]`` or
    ``[Hkv, D]``)."""
    import torch
    T = key.shape[0]
    _need(key, "key", torch.float16, (T, attn.kv_num_heads * attn.head_size))
    _need(value, "value", torch.float16, (T, attn.kv_num_heads * attn.head_size))  # None: latent
    lib = _lib.load()
    p = attn.c()
    kv = _kv(attn, key_cache, value_cache, block_table, cum, past, T, slot_mapping, k_scale,
             v_scale)
    c, s, rows, rd = _rot(attn, cos_cache, sin_cache)
    _check(lib.pa_append_kv(ctypes.byref(p), ctypes.byref(kv), key.data_ptr(), _ptr(value),
                            c, s, rows, rd, _stream(stream)))


def _workspace_bytes(lib, p, kv, routing, mq, mk) -> int:
    n = ctypes.c_size_t(0)
    if routing is None:
        _check(lib.pa_forward_workspace_bytes(ctypes.byref(p), ctypes.byref(kv), mq, mk,
                                              ctypes.byref(n)))
    else:
        r = routing.c()
        _check(lib.pa_forward_workspace_bytes_routed(ctypes.byref(p), ctypes.byref(kv),
                                                     ctypes.byref(r), mq, mk, ctypes.byref(n)))
    return int(n.value)


def forward_workspace_bytes(attn: Attn, key_cache, value_cache, block_table, cum, past,
                            token_count: int, max_query_len_bound: int = 0,
                            max_kv_len_bound: int = 0, k_scale=None, v_scale=None,
                            routing: Optional[Routing] = None) -> int:
    """``pa_forward_workspace_bytes`` (``..._routed`` with a forced ``routing``)."""
    lib = _lib.load()
    p = attn.c()
    kv = _kv(attn, key_cache, value_cache, block_table, cum, past, token_count,
             k_scale=k_scale, v_scale=v_scale)
    return _workspace_bytes(lib, p, kv, routing, max_query_len_bound, max_kv_len_bound)


def describe_plan(attn: Attn, key_cache, value_cache, block_table, cum, past, token_count: int,
                  max_query_len_bound: int = 0, max_kv_len_bound: int = 0, k_scale=None,
                  v_scale=None, routing: Optional[Routing] = None) -> str:
    lib = _lib.load()
    p = attn.c()
    kv = _kv(attn, key_cache, value_cache, block_table, cum, past, token_count,
             k_scale=k_scale, v_scale=v_scale)
    buf = ctypes.create_string_buffer(512)
    r = None if routing is None else ctypes.byref(routing.c())
    _check(lib.pa_describe_plan(ctypes.byref(p), ctypes.byref(kv), r, max_query_len_bound,
                                max_kv_len_bound, buf, 512))
    return buf.value.decode()


def forward(attn: Attn, query, key_cache, value_cache, block_table, cum, past, cos_cache=None,
            sin_cache=None, max_query_len_bound: int = 0, max_kv_len_bound: int = 0,
            workspace=None, out=None, stream=None, k_scale=None, v_scale=None,
            routing: Optional[Routing] = None):
    """``pa_forward``: attention output ``[T, H*DV]`` fp16 (``DV`` =
    ``attn.out_head_size``) for packed queries ``[T, H*D]``.  ``workspace``
    and ``out`` are allocated with torch when not given; quantized caches take
    ``k_scale``/``v_scale`` as for :func:`append_kv`.  A ``routing`` calls
    ``pa_forward_routed`` instead."""
    import torch
    T = query.shape[0]
    HD = attn.num_heads * attn.head_size
    HO = attn.num_heads * attn.out_head_size
    _need(query, "query", torch.float16, (T, HD))
    lib = _lib.load()
    p = attn.c()
    kv = _kv(attn, key_cache, value_cache, block_table, cum, past, T, k_scale=k_scale,
             v_scale=v_scale)
    if out is None:
        out = torch.empty((T, HO), dtype=torch.float16, device=query.device)
    _need(out, "out", torch.float16, (T, HO))
    need = _workspace_bytes(lib, p, kv, routing, max_query_len_bound, max_kv_len_bound)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr = _ptr(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c, s, rows, rd = _rot(attn, cos_cache, sin_cache)
    if routing is None:
        _check(lib.pa_forward(ctypes.byref(p), ctypes.byref(kv), query.data_ptr(), c, s, rows, rd,
                              max_query_len_bound, max_kv_len_bound, ws_ptr, ws_len,
                              out.data_ptr(), _stream(stream)))
    else:
        r = routing.c()
        _check(lib.pa_forward_routed(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(r),
                                     query.data_ptr(), c, s, rows, rd, max_query_len_bound,
                                     max_kv_len_bound, ws_ptr, ws_len, out.data_ptr(),
                                     _stream(stream)))
    return out


def forward_noalloc(attn: Attn, query, key_cache, value_cache, block_table, cum, past,
                    cos_cache=None, sin_cache=None, max_query_len_bound: int = 0,
                    max_kv_len_bound: int = 0, out=None, stream=None, k_scale=None,
                    v_scale=None):
    """``pa_forward_noalloc``: :func:`forward` on the library's own scratch
    array (no workspace argument; the library allocates nothing).  ``out``
    must be given by callers that allocate nothing themselves."""
    import torch
    T = query.shape[0]
    HD = attn.num_heads * attn.head_size
    HO = attn.num_heads * attn.out_head_size
    _need(query, "query", torch.float16, (T, HD))
    lib = _lib.load()
    p = attn.c()
    kv = _kv(attn, key_cache, value_cache, block_table, cum, past, T, k_scale=k_scale,
             v_scale=v_scale)
    if out is None:
        out = torch.empty((T, HO), dtype=torch.float16, device=query.device)
    _need(out, "out", torch.float16, (T, HO))
    c, s, rows, rd = _rot(attn, cos_cache, sin_cache)
    _check(lib.pa_forward_noalloc(ctypes.byref(p), ctypes.byref(kv), query.data_ptr(), c, s, rows,
                                  rd, max_query_len_bound, max_kv_len_bound, out.data_ptr(),
                                  _stream(stream)))
    return out


def timing_enable(max_launches: int) -> None:
    _check(_lib.load().pa_timing_enable(max_launches))


def timing_disable() -> None:
    _check(_lib.load().pa_timing_disable())


def stream_read(src, sink, stream=None) -> None:
    """``pa_bench_stream_read``: read every byte of the device tensor ``src``
    (a multiple of 16 KiB) once; ``sink`` is a device tensor of >= 4 bytes."""
    n = src.numel() * src.element_size()
    _check(_lib.load().pa_bench_stream_read(src.data_ptr(), n, sink.data_ptr(), _stream(stream)))


def timing_read(stage: str):
    """(total milliseconds, launches) recorded for ``stage`` in
    {append, decode, merge, prefill, plan, prefill_merge, q_norm}."""
    lib = _lib.load()
    ms = ctypes.c_double(0)
    n = ctypes.c_int32(0)
    _check(lib.pa_timing_read(_lib.STAGES[stage], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
