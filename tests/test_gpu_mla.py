"""GPU parity of latent attention (MLA; PagedAttention -- CUDA Design
Document, section 12) against the fp64 oracle: absorbed 576-channel rows
(512 latent + 64 rotary at offset 512), one kv head, V the leading 512
channels of K.  The appended K pool must be bit-exact (RoPE on the suffix
included) and every output row within 2e-3 of the oracle."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_append_amd import workloads as wl

from pa_harness import TOL, attn_for, max_err, split_routing

pytestmark = pytest.mark.gpu

LATENT = dict(kv_cache_layout=1, v_head_size=wl.MLA_V_HEAD_SIZE,
              rotary_offset=wl.MLA_ROTARY_OFFSET)


def device_inputs(w):
    """Device tensors with only the K pool (a latent cache has no V pool)."""
    import torch
    dev = wl.to_device(w, pools=False)
    kc = torch.empty(w.pool_shape(), dtype=torch.float16, device="cuda")

    def sink(start, arr):
        kc[start:start + arr.shape[0]].copy_(torch.from_numpy(arr))

    wl.fill_pool_chunks(w, wl.KIND_K, None, sink=sink)
    dev["key_cache"] = kc
    return dev


def gpu_latent(w, dev, **over):
    import torch
    import paged_kv_cache_append_amd as pa
    over, routing = split_routing(over)
    a = attn_for(w, **LATENT, **over)
    pa.append_kv(a, dev["key"], None, dev["key_cache"], None, dev["block_table"], dev["cum"],
                 dev["past"], dev["cos"], dev["sin"])
    out = pa.forward(a, dev["query"], dev["key_cache"], None, dev["block_table"], dev["cum"],
                     dev["past"], dev["cos"], dev["sin"], routing=routing)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def rot(w):
    return dict(cos_cache=w.cos_cache, sin_cache=w.sin_cache,
                rotary_interleaved=bool(w.rotary_interleaved), rotary_offset=wl.MLA_ROTARY_OFFSET)


def oracle_latent(w, kc, rows=None):
    nk, _ = oracle.append_kv(kc, None, w.key, None, w.cum, w.past, w.block_table,
                             kv_num_heads=1, head_size=w.head_size,
                             kv_cache_layout=oracle.LAYOUT_LATENT, **rot(w))
    ref = oracle.forward(w.query, nk, None, w.cum, w.past, w.block_table,
                         num_heads=w.num_heads, kv_num_heads=1, head_size=w.head_size,
                         scale=w.scale, softcap=w.softcap, local_window_size=w.local_window_size,
                         kv_cache_layout=oracle.LAYOUT_LATENT, v_head_size=wl.MLA_V_HEAD_SIZE,
                         rows=rows, **rot(w))
    return nk, ref


def check(w, **over):
    print(f"\n[mla] {w.name} B={w.batch_size} T={w.token_count} H={w.num_heads} "
          f"bs={w.block_size} W={w.local_window_size} softcap={w.softcap} "
          f"rot_inter={w.rotary_interleaved} {over}", flush=True)
    dev = device_inputs(w)
    out = gpu_latent(w, dev, **over)
    nk, ref = oracle_latent(w, w.pool_blocks(wl.KIND_K, range(w.num_blocks)))
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes(), "latent pool differs"
    err = max_err(out, ref)
    print(f"[mla] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("name", wl.MLA_CONFIG_NAMES)
def test_mla_scaled_configs(name):
    check(wl.scaled_down_mla(name))


def test_mla_chunked_prefill_rows_and_orphans():
    rng = np.random.default_rng(3401)
    w = wl._mla_case("mla_chunks", 3401, [1, 37, 1, 80], [500, 0, 1300, 64], 16, rng,
                     extra_tokens=3)
    check(w)


def test_mla_splits_are_merged():
    check(wl.scaled_down_mla("mla_decode_tp8"), split_tokens=64)


def test_mla_softcap_window_interleaved_rotary():
    rng = np.random.default_rng(3402)
    w = wl._mla_case("mla_features", 3402, [1, 9, 1], [700, 150, 40], 32, rng, block_size=16,
                     softcap=30.0, local_window_size=200, rotary_interleaved=1)
    check(w)


@pytest.mark.parametrize("name", wl.MLA_CONFIG_NAMES)
def test_mla_full_size_sampled(name):
    """The full workload on the GPU; the oracle checks the appended rows and
    a sample of 6 requests (the first, the longest, random others)."""
    w = wl.make_mla_workload(name)
    print(f"\n[mla] full {name} B={w.batch_size} H={w.num_heads}", flush=True)
    dev = device_inputs(w)
    out = gpu_latent(w, dev)
    kv = w.past + w.q_lens
    seqs = sorted({0, int(np.argmax(kv))} |
                  set(np.random.default_rng(5).choice(w.batch_size, 4, replace=False).tolist()))
    sub = wl.subset(w, seqs)
    sub.extra.update(latent=True)
    nk, ref = oracle_latent(sub, sub.pool_blocks(wl.KIND_K, range(sub.num_blocks)))
    gk = dev["key_cache"].cpu().numpy()
    ids = sub.extra["parent_block_ids"]
    assert np.array_equal(gk[ids], nk), "latent pool differs on the sampled requests"
    err = max_err(out[sub.extra["parent_rows"]], ref)
    print(f"[mla] sampled max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("heads", [64, 80])
def test_mla_shared_tile_head_groups(heads):
    """64+ heads: the four waves of a workgroup share one tile pair (shared
    mode); 80 heads leave three waves of the second group with no chunk of
    their own (they only copy)."""
    rng = np.random.default_rng(3403 + heads)
    w = wl._mla_case(f"mla_heads{heads}", 3403 + heads, [1, 1, 5, 1], [900, 33, 200, 2100],
                     heads, rng, softcap=25.0, local_window_size=1500, extra_tokens=2)
    check(w)


def test_mla_poisoned_pool():
    """Every slot no request has filled holds NaN: a read outside a row's
    admitted keys (or a masked key multiplied by zero) would show."""
    rng = np.random.default_rng(3404)
    w = wl._mla_case("mla_poison", 3404, [1, 3, 1], [70, 200, 1000], 64, rng, poison=True,
                     local_window_size=300)
    check(w)
    rng = np.random.default_rng(3405)
    w = wl._mla_case("mla_poison16", 3405, [1, 1, 4], [129, 4000, 63], 16, rng, poison=True)
    check(w, split_tokens=128)
