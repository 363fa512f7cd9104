"""Shared test plumbing: run a workload through the HIP library (via the
Python binding) and through the fp64 oracle, on the same host arrays."""
from __future__ import annotations

import numpy as np

import oracle
from paged_kv_cache_append_amd import workloads as wl

TOL = 2e-3   # max-abs error of fp16 outputs against the fp64 oracle


ROUTING_KEYS = ("path", "split_tokens", "prefill_pieces", "prefill_kernel")


def split_routing(over):
    """(attribute overrides, forced Routing or None) from one keyword dict:
    the routing keys go to ``pa_routing`` (include/pa_testing.h)."""
    import paged_kv_cache_append_amd as pa
    over = dict(over)
    r = {k: over.pop(k) for k in ROUTING_KEYS if k in over}
    r = {k: v for k, v in r.items() if v}
    return over, (pa.Routing(**r) if r else None)


def attn_for(w, **over):
    import paged_kv_cache_append_amd as pa
    assert not set(over) & set(ROUTING_KEYS), "routing goes through split_routing"
    a = pa.Attn(num_heads=w.num_heads, kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                block_size=w.block_size, scale=w.scale, softcap=w.softcap,
                local_window_size=w.local_window_size, do_rotary=w.do_rotary,
                rotary_interleaved=w.rotary_interleaved)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def gpu_append(w, dev, **over):
    import paged_kv_cache_append_amd as pa
    a = attn_for(w, **split_routing(over)[0])
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"])


def gpu_forward(w, dev, mq=0, mk=0, **over):
    import paged_kv_cache_append_amd as pa
    over, routing = split_routing(over)
    a = attn_for(w, **over)
    return pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                      dev["cum"], dev["past"], dev["cos"], dev["sin"], max_query_len_bound=mq,
                      max_kv_len_bound=mk, routing=routing)


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


# ---- quantized caches ------------------------------------------------------

def quant_inputs(w, cache_dtype, k_quant, v_quant, seed=7):
    """Drawn fp32 scales of both caches (host arrays)."""
    ks = wl.draw_scales(w, wl.KIND_K, cache_dtype, k_quant, seed)
    vs = wl.draw_scales(w, wl.KIND_V, cache_dtype, v_quant, seed)
    return ks, vs


def quant_kw(cache_dtype, k_quant, v_quant, ks, vs):
    return dict(cache_dtype=cache_dtype, k_quant_type=k_quant, v_quant_type=v_quant,
                k_scale=ks, v_scale=vs)


def gpu_quant_step(w, cache_dtype, k_quant, v_quant, ks, vs, slot_mapping=None, **over):
    """Quantized append + forward on the device: (device dict, fp16 out)."""
    import torch
    import paged_kv_cache_append_amd as pa
    dev = wl.to_device(w, cache_dtype=cache_dtype)
    dev["k_scale"] = torch.from_numpy(ks).cuda()
    dev["v_scale"] = torch.from_numpy(vs).cuda()
    over, routing = split_routing(over)
    a = attn_for(w, cache_dtype=cache_dtype, k_quant_type=k_quant, v_quant_type=v_quant, **over)
    sm = None if slot_mapping is None else torch.from_numpy(slot_mapping).cuda()
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"],
                 slot_mapping=sm, k_scale=dev["k_scale"], v_scale=dev["v_scale"])
    out = pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                     dev["cum"], dev["past"], dev["cos"], dev["sin"], k_scale=dev["k_scale"],
                     v_scale=dev["v_scale"], routing=routing)
    torch.cuda.synchronize()
    return dev, out.cpu().numpy()


def oracle_append_quant(w, cache_dtype, k_quant, v_quant, ks, vs, slot_mapping=None):
    kc = w.code_blocks(wl.KIND_K, range(w.num_blocks), cache_dtype)
    vc = w.code_blocks(wl.KIND_V, range(w.num_blocks), cache_dtype)
    return oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, w.block_table,
                            kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                            slot_mapping=slot_mapping,
                            **quant_kw(cache_dtype, k_quant, v_quant, ks, vs), **rot_kw(w))


def oracle_forward_quant(w, nk, nv, cache_dtype, k_quant, v_quant, ks, vs, rows=None):
    return oracle.forward(w.query, nk, nv, w.cum, w.past, w.block_table,
                          num_heads=w.num_heads, kv_num_heads=w.kv_num_heads,
                          head_size=w.head_size, scale=w.scale, softcap=w.softcap,
                          local_window_size=w.local_window_size, rows=rows,
                          **quant_kw(cache_dtype, k_quant, v_quant, ks, vs), **rot_kw(w))
