"""The benchmark workloads are the seeded synthetic inputs the measurement
plan specifies: config Cn is drawn from default_rng(1000 + n), and its
realised lengths, pool and table sizes are pinned here.  CPU only."""
import numpy as np
import pytest

from paged_kv_cache_append_amd import workloads as wl

# (name, seed, decode requests, sum of decode kv lengths, blocks used, pool, max blocks per row)
REALISED = [
    ("tiny_decode", 1001, 2, 38 + 51, 7, 16, 8),
    ("llama3_8b_mixed", 1002, 64, 128_772, 8_203, 9_024, 254),
    ("decode_heavy_256", 1003, 256, 2_218_308, 69_453, 76_399, 510),
    ("gemma2_prefill_window", 1004, 0, 0, 2_048, 2_253, 256),
    ("long_context_decode_rope", 1005, 8, 162_421, 2_541, 2_796, 2_049),
]


@pytest.mark.parametrize("name,seed,n_dec,kv_sum,used,pool,maxblk", REALISED)
def test_realised_sizes(name, seed, n_dec, kv_sum, used, pool, maxblk):
    w = wl.make_workload(name)
    kv = w.past.astype(np.int64) + w.q_lens
    dec = w.q_lens == 1
    assert w.seed == seed
    assert int(dec.sum()) == n_dec
    assert int(kv[dec].sum()) == kv_sum
    assert int(((kv + w.block_size - 1) // w.block_size).sum()) == used
    assert w.num_blocks == pool
    assert w.max_blocks_per_seq == maxblk


def test_tiny_table_is_the_config_permutation():
    w = wl.make_workload("tiny_decode")
    assert sorted(w.block_table.reshape(-1).tolist()) == list(range(16))
    assert w.block_table.shape == (2, 8)
    assert [int(x) for x in w.past] == [37, 50]


def test_cos_rows_of_the_rotary_workload():
    w = wl.make_workload("long_context_decode_rope")
    assert w.rotary_rows == 2_049 * 64 == 131_136
    assert w.cos_cache[0, 0] == np.float16(1.0) and w.sin_cache[0, 5] == np.float16(0.0)


def test_unmapped_and_shared_variants_poison_only_dead_blocks():
    w = wl.scaled_down("llama3_8b_mixed")
    ent = wl.random_unmapped_entries(w, 5, 0.3)
    assert ent, "the draw should unmap something"
    u = wl.with_unmapped_blocks(w, ent)
    for b, i in ent:
        assert u.block_table[b, i] == -1
    dead = sorted(u.extra["dead_blocks"])
    live = {int(x) for x in u.block_table.reshape(-1) if x >= 0}
    assert dead and not (set(dead) & live)
    assert np.all(np.isnan(u.pool_blocks(wl.KIND_K, dead).astype(np.float32)))
    assert np.all(np.isfinite(u.pool_blocks(wl.KIND_V, sorted(live)).astype(np.float32)))
    s = wl.with_shared_prefix(w, [(1, 2, 3)])
    assert np.array_equal(s.block_table[2, :3], w.block_table[1, :3])
    assert int(w.block_table[2, 0]) in s.extra["dead_blocks"]
    with pytest.raises(ValueError):
        wl.with_shared_prefix(w, [(0, 1, 1)])     # request 0 has only 15 cached positions
