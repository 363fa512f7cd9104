"""GPU parity of the attention sink (head_sink / smooth softmax,
PagedAttention -- CUDA Design Document, section 6) and of QK-Norm (section 7)
against the fp64 oracle.

The V pool must be bit-exact.  The normalized K pool is compared in fp16
units in the last place: the kernels reduce the sum of squares in fp32 (as
section 7.1 asks) and the oracle in fp64, so a value that lies next to an
fp16 rounding boundary may round the other way (one unit; RoPE after the
norm can carry that to two); the page itself compares its cache with the
same slack (section 8.7, implementation note P3).  The unit is taken at the
larger of the value and the row's RMS (1 after the norm): a rotated value
near zero inherits the absolute error of its O(1) inputs.  Outputs are within 2e-3
of the oracle's attention over the oracle's own pool."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_append_amd import workloads as wl

from pa_harness import TOL, attn_for, max_err, rot_kw, split_routing

pytestmark = pytest.mark.gpu


def extras(w, sink=True, norm=True, smooth=False, seed=5):
    rng = np.random.default_rng([seed, w.num_heads, w.head_size])
    e = {}
    if sink:
        e["head_sink"] = rng.uniform(-2.0, 3.0, w.num_heads).astype(np.float16)
    if smooth:
        e["use_smooth_softmax"] = 1
    if norm:
        e["q_norm_weight"] = rng.uniform(0.5, 1.5, w.head_size).astype(np.float16)
        e["k_norm_weight"] = rng.uniform(0.5, 1.5, w.head_size).astype(np.float16)
        e["qk_norm_epsilon"] = 1e-6
    return e


def run(w, e, path=0, quant=None, **over):
    import torch
    import paged_kv_cache_append_amd as pa
    print(f"\n[sink/norm] {w.name} T={w.token_count} H={w.num_heads} Hkv={w.kv_num_heads} "
          f"D={w.head_size} path={path} sink={'head_sink' in e} smooth={e.get('use_smooth_softmax', 0)} "
          f"norm={'q_norm_weight' in e} quant={quant} {over}", flush=True)
    cd = quant[0] if quant else wl.CACHE_FP16
    dev = wl.to_device(w, cache_dtype=cd)
    t = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in e.items()}
    sc = {}
    qkw = {}
    if quant:
        cd, kq, vq = quant
        ks = wl.draw_scales(w, wl.KIND_K, cd, kq, 7)
        vs = wl.draw_scales(w, wl.KIND_V, cd, vq, 7)
        sc = dict(k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda())
        qkw = dict(cache_dtype=cd, k_quant_type=kq, v_quant_type=vq, k_scale=ks, v_scale=vs)
        over = dict(over, cache_dtype=cd, k_quant_type=kq, v_quant_type=vq)
    over, routing = split_routing(dict(over, path=path))
    a = attn_for(w, **t, **over)
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"], **sc)
    out = pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                     dev["cum"], dev["past"], dev["cos"], dev["sin"], routing=routing, **sc)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    if quant:
        kc = w.code_blocks(wl.KIND_K, range(w.num_blocks), cd)
        vc = w.code_blocks(wl.KIND_V, range(w.num_blocks), cd)
    else:
        kc = w.pool_blocks(wl.KIND_K, range(w.num_blocks))
        vc = w.pool_blocks(wl.KIND_V, range(w.num_blocks))
    norm = {}
    if "k_norm_weight" in e:
        norm = dict(k_norm_weight=e["k_norm_weight"], qk_norm_epsilon=1e-6)
    nk, nv = oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, w.block_table,
                              kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                              **rot_kw(w), **norm, **qkw)
    gk = dev["key_cache"].cpu().numpy()
    gv = dev["value_cache"].cpu().numpy()
    assert np.array_equal(gv, nv), "value pool differs from the oracle append"
    if quant:
        if cd == wl.CACHE_INT8:
            d = np.abs(gk.astype(np.int32) - nk.astype(np.int32))
        else:
            d = ulps_fp8(gk, nk)
        assert d.max() <= 1, f"key codes differ by {d.max()}"
    elif norm:
        diff = np.abs(gk.astype(np.float64) - nk.astype(np.float64))
        unit = np.spacing(np.maximum(np.abs(nk.astype(np.float64)), 1.0).astype(np.float16))
        d = diff / unit.astype(np.float64)
        frac = np.count_nonzero(diff) / diff.size
        print(f"[sink/norm] K pool: max {d.max():.2f} units (max abs {diff.max():.2e}), "
              f"{frac:.2e} of elements differ", flush=True)
        assert d.max() <= 2 and frac < 1e-2
    else:
        assert np.array_equal(gk, nk), "key pool differs from the oracle append"
    fw = dict(head_sink=e.get("head_sink"), use_smooth_softmax=bool(e.get("use_smooth_softmax")))
    if "q_norm_weight" in e:
        fw.update(q_norm_weight=e["q_norm_weight"], qk_norm_epsilon=1e-6)
    ref = oracle.forward(w.query, nk, nv, w.cum, w.past, w.block_table, num_heads=w.num_heads,
                         kv_num_heads=w.kv_num_heads, head_size=w.head_size, scale=w.scale,
                         softcap=w.softcap, local_window_size=w.local_window_size, **rot_kw(w),
                         **fw, **qkw)
    err = max_err(out, ref)
    print(f"[sink/norm] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err


def ulps_fp8(a, b):
    """Distance of e4m3fn codes in steps of the format (sign-magnitude order)."""
    ia = np.where(a & 0x80, -(a.astype(np.int32) & 0x7F), a.astype(np.int32) & 0x7F)
    ib = np.where(b & 0x80, -(b.astype(np.int32) & 0x7F), b.astype(np.int32) & 0x7F)
    return np.abs(ia - ib)


@pytest.mark.parametrize("name", wl.CONFIG_NAMES)
@pytest.mark.parametrize("path", [0, 1, 2])
def test_sink_and_qk_norm_scaled_configs(name, path):
    w = wl.scaled_down(name)
    run(w, extras(w), path)


@pytest.mark.parametrize("name", ["llama3_8b_mixed", "gemma2_prefill_window"])
def test_sink_only_and_norm_only(name):
    w = wl.scaled_down(name)
    run(w, extras(w, sink=True, norm=False), 0)
    run(w, extras(w, sink=False, norm=True), 0)


def test_smooth_softmax():
    w = wl.scaled_down("llama3_8b_mixed")
    run(w, extras(w, sink=False, norm=False, smooth=True), 0)
    run(w, extras(w, sink=False, norm=False, smooth=True), 1)


def test_sink_through_decode_splits_and_prefill_pieces():
    # long rows: several decode splits (merge kernel) and prefill tiles cut
    # into pieces (prefill merge kernel)
    w = wl.build_case("sink_long", 3301, q_lens=[1, 1, 300, 1], past=[5000, 20, 4200, 3000],
                      num_heads=8, kv_num_heads=2, head_size=128, block_size=16, softcap=10.0)
    run(w, extras(w), 0, split_tokens=128)
    run(w, extras(w), 2, prefill_pieces=3)


@pytest.mark.parametrize("kernel", [1, 2, 3])
def test_sink_on_the_wide_head_prefill_kernels(kernel):
    w = wl.build_case("sink_wide", 3302, q_lens=[130, 67, 1], past=[200, 0, 900], num_heads=16,
                      kv_num_heads=8, head_size=256, block_size=16, softcap=50.0,
                      local_window_size=96, do_rotary=1, rotary_dim=64)
    run(w, extras(w), 2, prefill_kernel=kernel)


def test_sink_and_norm_with_a_quantized_pool():
    w = wl.scaled_down("decode_heavy_256")
    run(w, extras(w), 0, quant=(wl.CACHE_INT8, wl.QUANT_PER_CHANNEL, wl.QUANT_PER_TENSOR))
    w = wl.scaled_down("long_context_decode_rope")
    run(w, extras(w), 0, quant=(wl.CACHE_FP8, wl.QUANT_PER_TENSOR, wl.QUANT_PER_CHANNEL))


def test_sink_and_qk_norm_full_size_sampled():
    """llama3_8b_mixed at full size with a head sink and QK-Norm, as bench.py
    --head-sink --qk-norm times it (decode beside the prefill, automatic
    routing): the written V rows bit-exact and the normalized K rows within
    two fp16 units of the oracle's append, untouched blocks unchanged, and
    sampled decode requests and prefill rows against the oracle, recomputed
    one request at a time on a compact copy of its blocks."""
    import torch
    import paged_kv_cache_append_amd as pa
    from test_gpu_fullsize import sample_plan, touched_blocks
    w = wl.make_workload("llama3_8b_mixed")
    e = extras(w)
    print(f"\n[sink/norm] full {w.name} B={w.batch_size} T={w.token_count} "
          f"blocks={w.num_blocks}", flush=True)
    dev = wl.to_device(w)
    t = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in e.items()}
    a = attn_for(w, **t)
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"])
    out = pa.forward(a, dev["query"], dev["key_cache"], dev["value_cache"], dev["block_table"],
                     dev["cum"], dev["past"], dev["cos"], dev["sin"])
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    norm = dict(k_norm_weight=e["k_norm_weight"], qk_norm_epsilon=1e-6)

    ids = touched_blocks(w)
    remap = {old: new for new, old in enumerate(ids)}
    table = np.vectorize(lambda x: remap.get(int(x), 0))(w.block_table).astype(np.int32)
    nk, nv = oracle.append_kv(w.pool_blocks(wl.KIND_K, ids), w.pool_blocks(wl.KIND_V, ids),
                              w.key, w.value, w.cum, w.past, table,
                              kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                              **rot_kw(w), **norm)
    idx = torch.tensor(ids, device="cuda", dtype=torch.long)
    gk = dev["key_cache"].index_select(0, idx).cpu().numpy()
    assert dev["value_cache"].index_select(0, idx).cpu().numpy().tobytes() == nv.tobytes()
    diff = np.abs(gk.astype(np.float64) - nk.astype(np.float64))
    unit = np.spacing(np.maximum(np.abs(nk.astype(np.float64)), 1.0).astype(np.float16))
    units = diff / unit.astype(np.float64)
    print(f"[sink/norm] K rows of {len(ids)} written blocks: max {units.max():.2f} units, "
          f"{np.count_nonzero(diff) / diff.size:.2e} of elements differ", flush=True)
    assert units.max() <= 2 and np.count_nonzero(diff) / diff.size < 1e-2
    rng = np.random.default_rng(23)
    rest = sorted(set(range(w.num_blocks)) - set(ids))
    pick = sorted(int(x) for x in rng.choice(rest, size=min(64, len(rest)), replace=False))
    sel = torch.tensor(pick, device="cuda", dtype=torch.long)
    assert dev["key_cache"].index_select(0, sel).cpu().numpy().tobytes() == \
        w.pool_blocks(wl.KIND_K, pick).tobytes()
    del dev

    fw = dict(head_sink=e["head_sink"], q_norm_weight=e["q_norm_weight"], qk_norm_epsilon=1e-6)
    worst = 0.0
    for b, rows in sample_plan(w, rng):
        sub = wl.subset(w, [b])
        snk, snv = oracle.append_kv(sub.pool_blocks(wl.KIND_K, range(sub.num_blocks)),
                                    sub.pool_blocks(wl.KIND_V, range(sub.num_blocks)),
                                    sub.key, sub.value, sub.cum, sub.past, sub.block_table,
                                    kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                                    **rot_kw(sub), **norm)
        ref = oracle.forward(sub.query, snk, snv, sub.cum, sub.past, sub.block_table,
                             num_heads=w.num_heads, kv_num_heads=w.kv_num_heads,
                             head_size=w.head_size, scale=w.scale, softcap=w.softcap,
                             local_window_size=w.local_window_size, rows=rows,
                             **rot_kw(sub), **fw)
        prow = sub.extra["parent_rows"] if rows is None else sub.extra["parent_rows"][rows]
        err = max_err(out[prow], ref)
        print(f"[sink/norm] request {b} (past {int(w.past[b])}, q_len {int(w.q_lens[b])}) "
              f"rows {len(prow)}: max_abs_err={err:.3e}", flush=True)
        worst = max(worst, err)
    assert worst <= TOL, worst
