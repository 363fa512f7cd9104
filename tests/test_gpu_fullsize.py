"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (automatic routing, no bounds).  The append is checked
bit-exactly on every block that receives a new token and on a random sample
of untouched blocks; the forward on sampled rows (32 decode requests, and
the first and last 64 rows, the tile edges and drawn rows of every prefill
request), recomputed one request at a time by the fp64 oracle on a compact
copy of that request's blocks."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_append_amd import workloads as wl

from pa_harness import TOL, gpu_append, gpu_forward, max_err, oracle_append, oracle_forward

pytestmark = pytest.mark.gpu


def touched_blocks(w):
    ids = set()
    bs = w.block_size
    for b in range(w.batch_size):
        past, ql = int(w.past[b]), int(w.q_lens[b])
        for p in range(past, past + ql, 1):
            ids.add(int(w.block_table[b, p // bs]))
    return sorted(ids)


def sample_plan(w, rng, n_decode=32, edge_rows=64):
    """(request, rows within it) pairs to recompute with the oracle: up to
    ``n_decode`` decode requests (the longest, the shortest and drawn
    others), and for every prefill request its first and last
    ``edge_rows`` rows plus 16 drawn rows and the rows at the query-tile
    edges that fall between (tiles of 128 rows of (token, head) pairs, so
    128 / g tokens)."""
    ql = w.q_lens
    dec = [b for b in range(w.batch_size) if ql[b] == 1]
    pre = [b for b in range(w.batch_size) if ql[b] > 1]
    picks = []
    if dec:
        kv = w.past[dec]
        chosen = {dec[int(np.argmax(kv))], dec[int(np.argmin(kv))]}
        others = [b for b in dec if b not in chosen]
        k = min(max(0, n_decode - len(chosen)), len(others))
        chosen |= {int(x) for x in rng.choice(others, size=k, replace=False)}
        picks += [(b, None) for b in sorted(chosen)]
    g = w.num_heads // w.kv_num_heads
    tile = max(1, 128 // g)
    for b in pre:
        n = int(ql[b])
        rows = set(range(min(edge_rows, n))) | set(range(max(0, n - edge_rows), n))
        rows |= {int(x) for x in rng.integers(0, n, 16)}
        rows |= {r for t in range(tile, n, tile) for r in (t - 1, t) if r < n}
        picks.append((b, sorted(rows)))
    return picks


@pytest.mark.parametrize("name", wl.CONFIG_NAMES)
def test_full_size_workload(name):
    import torch
    w = wl.make_workload(name)
    print(f"\n[case] full {name}: B={w.batch_size} T={w.token_count} blocks={w.num_blocks}",
          flush=True)
    dev = wl.to_device(w)
    gpu_append(w, dev)
    out = gpu_forward(w, dev)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    rng = np.random.default_rng(99)

    # append: every block that receives a token, exactly
    ids = touched_blocks(w)
    remap = {old: new for new, old in enumerate(ids)}
    table = np.vectorize(lambda x: remap.get(int(x), 0))(w.block_table).astype(np.int32)
    kc = w.pool_blocks(wl.KIND_K, ids)
    vc = w.pool_blocks(wl.KIND_V, ids)
    rot = dict(cos_cache=w.cos_cache, sin_cache=w.sin_cache,
               rotary_interleaved=bool(w.rotary_interleaved)) if w.do_rotary else {}
    nk, nv = oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, table,
                              kv_num_heads=w.kv_num_heads, head_size=w.head_size, **rot)
    idx = torch.tensor(ids, device="cuda", dtype=torch.long)
    assert dev["key_cache"].index_select(0, idx).cpu().numpy().tobytes() == nk.tobytes()
    assert dev["value_cache"].index_select(0, idx).cpu().numpy().tobytes() == nv.tobytes()
    # ... and untouched blocks keep their bytes
    rest = sorted(set(range(w.num_blocks)) - set(ids))
    if rest:
        pick = sorted(int(x) for x in rng.choice(rest, size=min(64, len(rest)), replace=False))
        sel = torch.tensor(pick, device="cuda", dtype=torch.long)
        assert dev["key_cache"].index_select(0, sel).cpu().numpy().tobytes() == \
            w.pool_blocks(wl.KIND_K, pick).tobytes()
        assert dev["value_cache"].index_select(0, sel).cpu().numpy().tobytes() == \
            w.pool_blocks(wl.KIND_V, pick).tobytes()
    print(f"[case] append bit-exact on {len(ids)} written blocks", flush=True)

    # forward: sampled requests / rows
    worst = 0.0
    for b, rows in sample_plan(w, rng):
        sub = wl.subset(w, [b])
        snk, snv = oracle_append(sub)
        ref = oracle_forward(sub, snk, snv, rows=rows)
        prow = sub.extra["parent_rows"] if rows is None else sub.extra["parent_rows"][rows]
        e = max_err(out[prow], ref)
        print(f"[case] request {b} (past {int(w.past[b])}, q_len {int(w.q_lens[b])}) "
              f"rows {len(prow)}: max_abs_err={e:.3e}", flush=True)
        worst = max(worst, e)
    assert worst <= TOL, worst


@pytest.mark.parametrize("name", ["gemma2_prefill_window", "llama3_8b_mixed"])
def test_full_size_slot_mapping(name):
    """The append with explicit write slots (scattered over the whole pool,
    5 % of the tokens given -1) at full size: both pools bit-exact against
    the oracle's append, then sampled forward rows against the oracle on
    those pools."""
    import torch
    import paged_kv_cache_append_amd as pa
    from pa_harness import attn_for, rot_kw
    w = wl.make_workload(name)
    sm = wl.random_slot_mapping(w, 4242, skip_fraction=0.05)
    print(f"\n[case] full {name} with slot_mapping: T={w.token_count} "
          f"skipped={int((sm < 0).sum())}", flush=True)
    dev = wl.to_device(w)
    pa.append_kv(attn_for(w), dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"],
                 slot_mapping=torch.from_numpy(sm).cuda())
    out = gpu_forward(w, dev)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    kc = w.pool_blocks(wl.KIND_K, range(w.num_blocks))
    vc = w.pool_blocks(wl.KIND_V, range(w.num_blocks))
    nk, nv = oracle.append_kv(kc, vc, w.key, w.value, w.cum, w.past, w.block_table,
                              kv_num_heads=w.kv_num_heads, head_size=w.head_size,
                              slot_mapping=sm, **rot_kw(w))
    del kc, vc
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes()
    assert dev["value_cache"].cpu().numpy().tobytes() == nv.tobytes()
    print("[case] append bit-exact on the whole pools", flush=True)
    rng = np.random.default_rng(7)
    rows = sorted(int(x) for x in rng.choice(w.token_count, size=min(24, w.token_count),
                                             replace=False))
    ref = oracle.forward(w.query, nk, nv, w.cum, w.past, w.block_table, num_heads=w.num_heads,
                         kv_num_heads=w.kv_num_heads, head_size=w.head_size, scale=w.scale,
                         softcap=w.softcap, local_window_size=w.local_window_size, rows=rows,
                         **rot_kw(w))
    e = max_err(out[rows], ref)
    print(f"[case] {len(rows)} sampled rows: max_abs_err={e:.3e}", flush=True)
    assert e <= TOL, e
