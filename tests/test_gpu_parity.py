"""GPU parity of the HIP path against the fp64 oracle on sizes the oracle
finishes in seconds (several tiles, ragged tails): the append must be
bit-exact (the whole pool, written and untouched slots) and every output row
within 2e-3 max-abs of the oracle.  Each case runs on the three routings of
pa_forward (automatic, decode kernel for every token, decode + prefill)."""
import numpy as np
import pytest

from paged_kv_cache_append_amd import workloads as wl

from pa_harness import (TOL, gpu_forward, gpu_step, max_err, oracle_append, oracle_append_slots,
                        oracle_forward)

pytestmark = pytest.mark.gpu

PATHS = [0, 1, 2]


def check(w, path=0, rows=None, **over):
    print(f"\n[case] {w.name} B={w.batch_size} T={w.token_count} H={w.num_heads} "
          f"Hkv={w.kv_num_heads} D={w.head_size} bs={w.block_size} W={w.local_window_size} "
          f"softcap={w.softcap} rot={w.do_rotary}/{w.rotary_interleaved} path={path} {over}",
          flush=True)
    dev, out = gpu_step(w, path=path, **over)
    nk, nv = oracle_append(w)
    gk = dev["key_cache"].cpu().numpy()
    gv = dev["value_cache"].cpu().numpy()
    assert gk.tobytes() == nk.tobytes(), "key pool differs from the oracle append"
    assert gv.tobytes() == nv.tobytes(), "value pool differs from the oracle append"
    ref = oracle_forward(w, nk, nv)
    err = max_err(out, ref)
    print(f"[case] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err
    return out, ref


@pytest.mark.parametrize("name", wl.CONFIG_NAMES)
@pytest.mark.parametrize("path", PATHS)
def test_scaled_configs(name, path):
    check(wl.scaled_down(name), path)


SWEEP = [
    # q_lens, past, H, Hkv, D, bs, extra kwargs
    ([1, 1, 1], [0, 15, 40], 8, 8, 64, 16, {}),                          # MHA (g = 1)
    ([1, 1], [16, 17], 8, 1, 64, 16, {}),                                # MQA (g = 8)
    ([5, 17], [0, 0], 4, 2, 128, 16, {}),                                # fresh prefill
    ([5, 2, 17], [1, 16, 40], 4, 2, 64, 32, {}),                         # chunked prefill
    ([17, 1, 0, 2], [15, 3, 9, 0], 4, 4, 64, 16, {}),                    # ragged, q_len 0
    ([9, 1], [20, 33], 4, 2, 128, 16, dict(local_window_size=5)),
    ([130, 1, 3], [300, 1000, 64], 6, 2, 256, 16,                        # g = 3 (chunks of 1)
     dict(local_window_size=200, softcap=5.0)),
    ([1, 1, 1, 1, 1], [900, 1, 77, 600, 2], 24, 2, 128, 16, dict(softcap=1.0)),   # g = 12
    ([3, 1, 40], [70, 129, 0], 8, 2, 64, 16,
     dict(do_rotary=1, rotary_interleaved=1, rotary_dim=32)),
    ([3, 1, 40], [70, 129, 0], 8, 2, 64, 16, dict(do_rotary=1, rotary_dim=20)),
    ([200], [0], 2, 1, 64, 64, dict(local_window_size=1)),
    ([1, 1, 1, 70], [5000, 20, 0, 3000], 8, 2, 64, 16, {}),              # several splits
    ([64, 1], [4000, 7000], 16, 8, 256, 16, dict(local_window_size=4096, softcap=50.0)),
    ([33, 2, 1], [1, 2, 3], 32, 8, 128, 128, dict(scale=0.3)),
    ([100, 1], [9000, 4000], 8, 2, 128, 16, {}),        # long keys, few tiles: auto pieces
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
@pytest.mark.parametrize("path", PATHS)
def test_sweep(case, path):
    q_lens, past, H, Hkv, D, bs, kw = SWEEP[case]
    w = wl.build_case(f"sweep{case}", 500 + case, q_lens=q_lens, past=past, num_heads=H,
                      kv_num_heads=Hkv, head_size=D, block_size=bs, **kw)
    check(w, path)


@pytest.mark.parametrize("path", PATHS)
def test_poisoned_pool(path):
    """Every slot the runtime has not filled is NaN (and unused blocks are
    NaN): reading any key past a request's length, or weighting a NaN value
    row by zero, shows up as a non-finite or wrong output."""
    w = wl.build_case("poison", 77, q_lens=[1, 9, 1, 33], past=[45, 17, 300, 0], num_heads=8,
                      kv_num_heads=2, head_size=128, block_size=16, extra_blocks_per_seq=2,
                      poison=True, softcap=20.0)
    check(w, path)


@pytest.mark.parametrize("path", [0, 2])
def test_tokens_owned_by_no_request(path):
    w = wl.build_case("orphans", 78, q_lens=[2, 1, 5], past=[10, 40, 0], num_heads=4,
                      kv_num_heads=2, head_size=64, block_size=16, extra_tokens=3)
    out, ref = check(w, path)
    assert np.all(out[-3:] == 0)


def test_split_length_changes_only_rounding():
    w = wl.build_case("splits", 79, q_lens=[1, 1, 1], past=[6000, 1500, 90], num_heads=8,
                      kv_num_heads=1, head_size=64, block_size=32)
    outs = [check(w, 1, split_tokens=st)[0] for st in (0, 64, 192, 1024, 8192)]
    for o in outs[1:]:
        assert np.max(np.abs(o.astype(np.float64) - outs[0])) <= 1e-3


PIECE_CASES = [
    # q_lens, past, H, Hkv, D, bs, extra kwargs: prefill tiles whose key range
    # spans several 64-key tiles, cut into 1..4 pieces merged on the device
    ([130, 1, 77], [500, 900, 0], 8, 2, 128, 16, {}),
    ([64, 3], [1500, 40], 16, 8, 256, 16, dict(local_window_size=700, softcap=50.0)),
    ([200, 9], [300, 0], 8, 1, 64, 32, dict(do_rotary=1, rotary_dim=64)),
]


@pytest.mark.parametrize("case", range(len(PIECE_CASES)))
@pytest.mark.parametrize("pieces", [1, 2, 3, 4])
def test_prefill_pieces(case, pieces):
    """Every split of a prefill tile's key range over workgroups matches the
    oracle (the pieces only change the summation order)."""
    q_lens, past, H, Hkv, D, bs, kw = PIECE_CASES[case]
    w = wl.build_case(f"pieces{case}", 600 + case, q_lens=q_lens, past=past, num_heads=H,
                      kv_num_heads=Hkv, head_size=D, block_size=bs, **kw)
    check(w, 2, prefill_pieces=pieces)


def test_bounds_do_not_change_results():
    """No bounds, tight bounds and loose bounds give bitwise-identical output
    (bounds only size launches and workspace)."""
    import torch
    w = wl.build_case("bounds", 80, q_lens=[1, 1, 20, 1], past=[3000, 10, 700, 1200], num_heads=8,
                      kv_num_heads=2, head_size=128, block_size=16)
    dev, base = gpu_step(w, path=2)
    mq = int(w.q_lens.max())
    mk = int((w.past + w.q_lens).max())
    for bq, bk in ((mq, mk), (10 * mq, 10 * mk), (0, mk), (mq, 0)):
        o = gpu_forward(w, dev, mq=bq, mk=bk, path=2)
        torch.cuda.synchronize()
        assert o.cpu().numpy().tobytes() == base.tobytes(), (bq, bk)


def test_batch_order_permutation():
    w = wl.build_case("perm", 81, q_lens=[1, 7, 1, 3], past=[100, 30, 5, 64], num_heads=4,
                      kv_num_heads=2, head_size=64, block_size=16)
    _, out = gpu_step(w, path=2)
    order = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(w.cum[b], w.cum[b + 1]) for b in order])
    w2 = wl.build_case("perm", 81, q_lens=[1, 7, 1, 3], past=[100, 30, 5, 64], num_heads=4,
                       kv_num_heads=2, head_size=64, block_size=16)
    w2.cum = np.concatenate([[0], np.cumsum(w.q_lens[order])]).astype(np.int32)
    w2.past = w.past[order].copy()
    w2.block_table = w.block_table[order].copy()
    w2.query, w2.key, w2.value = w.query[rows], w.key[rows], w.value[rows]
    _, out2 = gpu_step(w2, path=2)
    assert np.max(np.abs(out2.astype(np.float64) - out[rows])) <= 1e-3


WIDE_CASES = [
    # q_lens, past, H, Hkv, D = 256, bs, extra kwargs: the prefill kernels of
    # the 256-channel head (4 waves x 32 rows, 8 waves x 16 rows, 8 waves x 32
    # rows)
    ([130, 1, 3], [300, 1000, 64], 6, 2, 256, 16, dict(local_window_size=200, softcap=5.0)),
    ([64, 1], [4000, 7000], 16, 8, 256, 16, dict(local_window_size=4096, softcap=50.0)),
    ([257, 2, 40], [0, 129, 3000], 8, 4, 256, 32, {}),
    ([70, 5], [16, 200], 4, 1, 256, 64, dict(do_rotary=1, rotary_dim=128, local_window_size=33)),
]


@pytest.mark.parametrize("case", range(len(WIDE_CASES)))
@pytest.mark.parametrize("kernel", [1, 2, 3])
def test_wide_head_prefill_kernels(case, kernel):
    q_lens, past, H, Hkv, D, bs, kw = WIDE_CASES[case]
    w = wl.build_case(f"wide{case}", 700 + case, q_lens=q_lens, past=past, num_heads=H,
                      kv_num_heads=Hkv, head_size=D, block_size=bs, **kw)
    check(w, 2, prefill_kernel=kernel)


@pytest.mark.parametrize("kernel", [1, 2, 3])
def test_wide_head_prefill_kernels_with_pieces(kernel):
    q_lens, past, H, Hkv, D, bs, kw = PIECE_CASES[1]
    w = wl.build_case("pieces1", 601, q_lens=q_lens, past=past, num_heads=H,
                      kv_num_heads=Hkv, head_size=D, block_size=bs, **kw)
    check(w, 2, prefill_kernel=kernel, prefill_pieces=3)


def many_requests_case(D, seed):
    # 40 requests: decode rows between prefill chunks of 2..200 tokens, so the
    # prefill tile order groups several requests with unequal tile counts
    rng = np.random.default_rng(seed)
    q_lens = [int(x) if rng.random() < 0.7 else 1 for x in rng.integers(2, 201, size=40)]
    past = [int(x) for x in rng.integers(0, 501, size=40)]
    return wl.build_case(f"many{D}", seed, q_lens=q_lens, past=past, num_heads=8,
                         kv_num_heads=2, head_size=D, block_size=16,
                         **(dict(local_window_size=300, softcap=30.0) if D == 256 else {}))


@pytest.mark.parametrize("kernel", [1, 2, 3])
def test_prefill_tile_order_over_many_requests(kernel):
    check(many_requests_case(256, 960), 2, prefill_kernel=kernel)


def test_prefill_tile_order_over_many_requests_d128():
    check(many_requests_case(128, 961), 2)


SLOT_CASES = [
    # q_lens, past, H, Hkv, D, bs, extra kwargs, fraction of tokens with -1
    ([1, 1, 40, 3], [50, 900, 0, 64], 8, 2, 64, 16, {}, 0.25),
    ([130, 1], [300, 1000], 6, 2, 128, 32, dict(do_rotary=1, rotary_dim=128), 0.1),
    ([64, 2], [100, 3000], 16, 8, 256, 16,
     dict(do_rotary=1, rotary_interleaved=1, rotary_dim=64, softcap=50.0), 0.0),
]


@pytest.mark.parametrize("case", range(len(SLOT_CASES)))
def test_slot_mapping(case):
    """Explicit write slots (scattered over the whole pool, some -1): the
    pools match the oracle's append bit for bit and the forward, which reads
    through the block table as always, matches the oracle."""
    import torch
    import paged_kv_cache_append_amd as pa
    from pa_harness import attn_for
    q_lens, past, H, Hkv, D, bs, kw, skip = SLOT_CASES[case]
    w = wl.build_case(f"slots{case}", 900 + case, q_lens=q_lens, past=past, num_heads=H,
                      kv_num_heads=Hkv, head_size=D, block_size=bs, extra_tokens=2, **kw)
    sm = wl.random_slot_mapping(w, 77 + case, skip_fraction=skip)
    print(f"\n[case] slot_mapping {w.name} T={w.token_count} D={D} skipped={int((sm < 0).sum())}",
          flush=True)
    dev = wl.to_device(w)
    a = attn_for(w)
    pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                 dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"],
                 slot_mapping=torch.from_numpy(sm).cuda())
    out = gpu_forward(w, dev)
    torch.cuda.synchronize()
    nk, nv = oracle_append_slots(w, sm)
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes()
    assert dev["value_cache"].cpu().numpy().tobytes() == nv.tobytes()
    err = max_err(out.cpu().numpy(), oracle_forward(w, nk, nv))
    print(f"[case] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err


def test_slot_mapping_prefix_cache_hit():
    """A chunked prefill whose first tokens are already cached: one append
    of the cached tokens, then the chunk's append with those tokens given
    -1, leaves the device pool and output bit-identical to one derived
    append."""
    import torch
    import oracle
    import paged_kv_cache_append_amd as pa
    from pa_harness import attn_for
    w = wl.build_case("prefix", 950, q_lens=[70, 1, 33], past=[0, 400, 16], num_heads=8,
                      kv_num_heads=2, head_size=128, block_size=16, do_rotary=1, rotary_dim=64)
    derived = np.full(w.token_count, -1, np.int32)
    for t in range(w.token_count):
        b, j = oracle.locate_token(w.cum, t)
        blk, off = oracle.derived_slot(w.block_table, b, oracle.token_position(w.past, b, j),
                                       w.block_size)
        derived[t] = blk * w.block_size + off
    k = 40
    first = np.where(np.arange(w.token_count) < k, derived, -1).astype(np.int32)
    rest = np.where(np.arange(w.token_count) < k, -1, derived).astype(np.int32)
    a = attn_for(w)
    dev = wl.to_device(w)
    for sm in (first, rest):
        pa.append_kv(a, dev["key"], dev["value"], dev["key_cache"], dev["value_cache"],
                     dev["block_table"], dev["cum"], dev["past"], dev["cos"], dev["sin"],
                     slot_mapping=torch.from_numpy(sm).cuda())
    out = gpu_forward(w, dev).cpu().numpy()
    ref_dev, ref_out = gpu_step(w)
    assert dev["key_cache"].cpu().numpy().tobytes() == ref_dev["key_cache"].cpu().numpy().tobytes()
    assert dev["value_cache"].cpu().numpy().tobytes() == \
        ref_dev["value_cache"].cpu().numpy().tobytes()
    assert out.tobytes() == ref_out.tobytes()
