"""GPU parity for unmapped blocks, shared prefix blocks and the rolling
sliding-window cache (PagedAttention -- CUDA Design Document, §9.2 item 3,
§9.3 and the paging tests of §17.2), against the fp64 oracle.

A -1 table entry is an unmapped block: its positions are masked out of the
softmax, the derived append writes nothing there, and a row left with no key
is 0.  The physical blocks such entries used to name are poisoned (NaN, or
the int8 code 127), so any read through a stale entry shows in the output.
Pools are compared byte for byte, outputs element-wise within 2e-3."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_append_amd import workloads as wl

from pa_harness import (TOL, attn_for, gpu_step, max_err, oracle_append, oracle_forward,
                        split_routing)

pytestmark = pytest.mark.gpu


def check(w, **over):
    print(f"\n[unmapped] {w.name} B={w.batch_size} T={w.token_count} D={w.head_size} "
          f"bs={w.block_size} W={w.local_window_size} holes="
          f"{int((w.block_table < 0).sum())} dead={len(w.extra.get('dead_blocks', ()))} {over}",
          flush=True)
    dev, out = gpu_step(w, **over)
    nk, nv = oracle_append(w)
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes(), "key pool differs"
    assert dev["value_cache"].cpu().numpy().tobytes() == nv.tobytes(), "value pool differs"
    ref = oracle_forward(w, nk, nv)
    err = max_err(out, ref)
    print(f"[unmapped] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err
    return out, ref


def holes_decode():
    """12 decode requests (D=128, bs=32): a drawn quarter of the cached
    blocks unmapped; request 0 fully unmapped (its new token's block too, so
    its row is 0); on the longest request, block indices 2 and 3 (positions
    64..127: one whole 64-token split) unmapped."""
    w = wl.scaled_down("decode_heavy_256")
    ent = set(wl.random_unmapped_entries(w, 11, 0.25))
    ent |= {(0, i) for i in range(int(w.past[0]) // w.block_size + 1)}
    longest = int(np.argmax(w.past))
    ent |= {(longest, 2), (longest, 3)}
    return wl.with_unmapped_blocks(w, sorted(ent))


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_unmapped_blocks_in_decode_splits(split_tokens):
    w = holes_decode()
    out, ref = check(w, split_tokens=split_tokens)
    assert np.all(out[0] == 0) and np.all(ref[0] == 0)


def holes_prefill():
    """Prefill tiles with holes: the windowed, softcapped D=256 case (bs=16,
    so a 64-key tile spans four blocks) with unmapped blocks inside the
    window of request 0 and a drawn quarter elsewhere."""
    w = wl.scaled_down("gemma2_prefill_window")
    ent = set(wl.random_unmapped_entries(w, 12, 0.25)) | {(0, 7), (0, 9), (0, 10)}
    return wl.with_unmapped_blocks(w, sorted(ent))


@pytest.mark.parametrize("kernel", [1, 2, 3])
@pytest.mark.parametrize("pieces", [0, 3])
def test_unmapped_blocks_in_prefill_tiles(kernel, pieces):
    check(holes_prefill(), path=2, prefill_kernel=kernel, prefill_pieces=pieces)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_unmapped_blocks_in_a_mixed_batch(path):
    w = wl.scaled_down("llama3_8b_mixed")
    ent = set(wl.random_unmapped_entries(w, 13, 0.3))
    # the 75 cached positions of the second prefill chunk: blocks 1 and 3 unmapped
    ent |= {(7, 1), (7, 3)}
    check(wl.with_unmapped_blocks(w, sorted(ent)), path=path)


def test_unmapped_blocks_with_rotary_and_many_splits():
    w = wl.scaled_down("long_context_decode_rope")
    ent = set(wl.random_unmapped_entries(w, 14, 0.2)) | {(0, i) for i in range(10, 20)}
    check(wl.with_unmapped_blocks(w, sorted(ent)), split_tokens=128)


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_positions_past_the_table_capacity(split_tokens):
    """A table narrower than a request needs: positions past its capacity
    read as unmapped, the new token past it is not written, and a row whose
    window lies wholly past it is 0 (request 0: position 2000, window 100,
    capacity 512 keys)."""
    w = wl.build_case("past_capacity", 3301, q_lens=[1, 1, 1], past=[2000, 500, 90],
                      num_heads=8, kv_num_heads=2, head_size=64, block_size=16,
                      local_window_size=100)
    w.block_table = np.ascontiguousarray(w.block_table[:, :32])
    out, ref = check(w, split_tokens=split_tokens)
    assert np.all(out[0] == 0) and np.all(ref[0] == 0)


@pytest.mark.parametrize("kernel", [1, 2, 3])
def test_prefill_positions_past_the_table_capacity(kernel):
    """Prefill rows whose causal range runs past the table's capacity (32
    blocks of 16 = 512 keys): the keys past it are unmapped and masked, and
    the new tokens there are not written.  Request 0 (positions 470..569)
    straddles the capacity, request 1 (600..629) lies wholly past it: with a
    window of 64 its rows have no key and are 0."""
    w = wl.build_case("past_capacity_prefill", 3303, q_lens=[100, 30, 1], past=[470, 600, 40],
                      num_heads=8, kv_num_heads=4, head_size=256, block_size=16,
                      local_window_size=64, softcap=30.0)
    w.block_table = np.ascontiguousarray(w.block_table[:, :32])
    out, ref = check(w, path=2, prefill_kernel=kernel)
    t1 = int(w.cum[1])
    assert np.all(ref[t1:t1 + 30] == 0) and np.all(out[t1:t1 + 30] == 0)


def test_unmapped_blocks_int8_pool():
    from pa_harness import gpu_quant_step, oracle_append_quant, oracle_forward_quant, quant_inputs
    w = holes_decode()
    I8, PC = wl.CACHE_INT8, wl.QUANT_PER_CHANNEL
    print(f"\n[unmapped] int8 {w.name} holes={int((w.block_table < 0).sum())}", flush=True)
    ks, vs = quant_inputs(w, I8, PC, PC)
    dev, out = gpu_quant_step(w, I8, PC, PC, ks, vs, split_tokens=64)
    nk, nv = oracle_append_quant(w, I8, PC, PC, ks, vs)
    assert np.array_equal(dev["key_cache"].cpu().numpy(), nk)
    assert np.array_equal(dev["value_cache"].cpu().numpy(), nv)
    ref = oracle_forward_quant(w, nk, nv, I8, PC, PC, ks, vs)
    err = max_err(out, ref)
    print(f"[unmapped] int8 max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err
    assert np.all(out[0] == 0)


def test_unmapped_blocks_latent():
    import torch
    from test_gpu_mla import device_inputs, gpu_latent, oracle_latent
    w = wl.scaled_down_mla("mla_decode_tp8")
    ent = set(wl.random_unmapped_entries(w, 15, 0.3))
    longest = int(np.argmax(w.past))
    ent |= {(longest, 1), (longest, 2)}
    w = wl.with_unmapped_blocks(w, sorted(ent))
    print(f"\n[unmapped] latent {w.name} holes={int((w.block_table < 0).sum())}", flush=True)
    dev = device_inputs(w)
    out = gpu_latent(w, dev, split_tokens=64)
    torch.cuda.synchronize()
    nk, ref = oracle_latent(w, w.pool_blocks(wl.KIND_K, range(w.num_blocks)))
    assert dev["key_cache"].cpu().numpy().tobytes() == nk.tobytes()
    err = max_err(out, ref)
    print(f"[unmapped] latent max_abs_err={err:.3e}", flush=True)
    assert err <= TOL, err


@pytest.mark.parametrize("path", [0, 2])
def test_shared_prefix_blocks(path):
    """Requests 1 and 2 of the mixed batch read the first blocks of request 4
    (read-only prefix sharing); their own former blocks are poisoned."""
    w = wl.scaled_down("llama3_8b_mixed")
    w = wl.with_shared_prefix(w, [(4, 1, 9), (4, 3, 8)])
    check(w, path=path)


# ---------------------------------------------------------------------------
# rolling sliding-window cache (§9.3): ring-buffer run vs full-cache run
# ---------------------------------------------------------------------------

def _rolling_gpu(ring, window, q_first, steps, H=8, Hkv=2, D=64, bs=16, maxblk=16, seed=21):
    """GPU outputs (fp16, host) of every step, and the oracle's of the last
    step, for the full cache (derived slots) or the ring-buffer cache
    (ceil(W/bs)+1 blocks per request, slot_mapping, evicted entries -1)."""
    import torch
    import paged_kv_cache_append_amd as pa
    B = len(q_first)
    if ring:
        alloc = wl.RingBlockAllocator(B, window, bs, maxblk, seed=5)
        nb = alloc.num_blocks
    else:
        table = wl.full_cache_table(B, maxblk, seed=5)
        nb = B * maxblk
    a = pa.Attn(num_heads=H, kv_num_heads=Hkv, head_size=D, block_size=bs, scale=0.2,
                local_window_size=window)
    kc = torch.zeros((nb, bs, Hkv, D), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    okc = np.zeros((nb, bs, Hkv, D), np.float16)
    ovc = np.zeros_like(okc)
    past = np.zeros(B, np.int32)
    outs = []
    ref = None
    for s in range(steps):
        q_lens = q_first if s == 0 else [1] * B
        cum, q, k, v = wl.step_tokens(seed, s, q_lens, H, Hkv, D)
        sm = None
        if ring:
            table, sm = alloc.step(past, q_lens)
        d = {n: torch.from_numpy(np.ascontiguousarray(x)).cuda()
             for n, x in (("q", q), ("k", k), ("v", v), ("cum", cum), ("past", past),
                          ("table", table))}
        smd = None if sm is None else torch.from_numpy(sm).cuda()
        pa.append_kv(a, d["k"], d["v"], kc, vc, d["table"], d["cum"], d["past"], slot_mapping=smd)
        out = pa.forward(a, d["q"], kc, vc, d["table"], d["cum"], d["past"])
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        okc, ovc = oracle.append_kv(okc, ovc, k, v, cum, past, table, kv_num_heads=Hkv,
                                    head_size=D, slot_mapping=sm)
        if s in (0, steps - 1):
            ref = oracle.forward(q, okc, ovc, cum, past, table, num_heads=H, kv_num_heads=Hkv,
                                 head_size=D, scale=0.2, local_window_size=window)
            err = max_err(outs[-1], ref)
            print(f"[rolling] ring={ring} step {s}: max_abs_err={err:.3e}", flush=True)
            assert err <= TOL, err
        past = past + np.asarray(q_lens, np.int32)
    return outs


@pytest.mark.parametrize("window", [40, 100])
def test_rolling_window_cache_bit_matches_full_cache(window):
    """Every decode step of the ring-buffer run is bit-identical to the
    full-cache run (§9.3.5); a mixed batch: one request past the window from
    the start, one crossing it during the run, one that never does."""
    print(f"\n[rolling] window {window}", flush=True)
    q_first = [window, window // 2, 1]
    full = _rolling_gpu(False, window, q_first, 90)
    ring = _rolling_gpu(True, window, q_first, 90)
    for s, (x, y) in enumerate(zip(full, ring)):
        assert x.tobytes() == y.tobytes(), f"step {s}"
