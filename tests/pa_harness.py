"""Shared test plumbing: run a workload through the HIP library (via the
Python binding) and through the fp64 oracle, on the same host arrays."""
from __future__ import annotations

import numpy as np

import oracle
from paged_kv_cache_append_amd import workloads as wl

TOL = 2e-3   # max-abs error of fp16 outputs against the fp64 oracle


def attn_for(w, **over):
    import paged_kv_cache_append_amd as pa
    a = pa.Attn(num_heads=w.num_heads, kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                block_size=w.block_size, scale=w.scale, softcap=w.softcap,
                local_window_size=w.local_window_size, do_rotary=w.do_rotary,
                rotary_interleaved=w.rotary_interleaved)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def gpu_append(w, dev, **over):
    import paged_kv_cache_append_amd as pa
    a = attn_for(w, **over)
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"])


def gpu_forward(w, dev, mq=0, mk=0, **over):
    import paged_kv_cache_append_amd as pa
    a = attn_for(w, **over)
    return pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                      dev["cum"], dev["past"], dev["cos"], dev["sin"], max_query_len_bound=mq,
                      max_kv_len_bound=mk)


def gpu_step(w, dev=None, **over):
    """append + forward on the device; returns (device dict, fp16 out as numpy)."""
    import torch
    dev = dev if dev is not None else wl.to_device(w)
    gpu_append(w, dev, **over)
    out = gpu_forward(w, dev, **over)
    torch.cuda.synchronize()
    return dev, out.cpu().numpy()


def rot_kw(w):
    if not w.do_rotary:
        return {}
    return dict(cos_cache=w.cos_cache, sin_cache=w.sin_cache,
                rotary_interleaved=bool(w.rotary_interleaved))


def oracle_append(w, kc=None, vc=None):
    kc = w.pool_blocks(wl.KIND_K, range(w.num_blocks)) if kc is None else kc
    vc = w.pool_blocks(wl.KIND_V, range(w.num_blocks)) if vc is None else vc
    return oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, w.block_table,
                            kv_num_heads=w.kv_num_heads, head_size=w.head_size, **rot_kw(w))


def oracle_append_slots(w, slot_mapping):
    kc = w.pool_blocks(wl.KIND_K, range(w.num_blocks))
    vc = w.pool_blocks(wl.KIND_V, range(w.num_blocks))
    return oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, w.block_table,
                            kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                            slot_mapping=slot_mapping, **rot_kw(w))


def oracle_forward(w, nk, nv, rows=None):
    return oracle.forward(w.query, nk, nv, w.cum, w.past, w.block_table,
                          num_heads=w.num_heads, kv_num_heads=w.kv_num_heads,
                          head_size=w.head_size, scale=w.scale, softcap=w.softcap,
                          local_window_size=w.local_window_size, rows=rows, **rot_kw(w))


def max_err(gpu16, ref64):
    g = gpu16.astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref64))) if g.size else 0.0
