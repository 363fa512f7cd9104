"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (automatic routing, no bounds).  The append is checked
bit-exactly on every block that receives a new token and on a random sample
of untouched blocks; the forward on sampled rows, recomputed one request at a
time by the fp64 oracle on a compact copy of that request's blocks."""
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


def sample_plan(w, rng):
    """(request, rows within it) pairs to recompute with the oracle."""
    ql = w.q_lens
    dec = [b for b in range(w.batch_size) if ql[b] == 1]
    pre = [b for b in range(w.batch_size) if ql[b] > 1]
    picks = []
    if dec:
        kv = w.past[dec]
        chosen = {dec[int(np.argmax(kv))], dec[int(np.argmin(kv))]}
        chosen |= {int(x) for x in rng.choice(dec, size=min(2, len(dec)), replace=False)}
        picks += [(b, None) for b in sorted(chosen)]
    for b in pre[:2]:
        n = int(ql[b])
        rows = sorted({0, 1, n - 1, n - 2} | {int(x) for x in rng.integers(0, n, 12)})
        picks.append((b, rows))
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
