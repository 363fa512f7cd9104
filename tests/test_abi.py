"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/pa.h and include/pa_testing.h, and rejects each malformed request with the status
and message the header documents (PagedAttention -- CUDA Design Document,
section 15: every violation names the offending argument).  No call here
reaches a HIP runtime function: only validation and host planning run."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_append_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # 16-byte aligned address, never dereferenced on the host

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libpa.so not built (run __graft_entry__.build())")


def header_functions(header="pa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^\s*(?:pa_status|size_t|const char \*)\s*(pa_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    assert set(header_functions()) >= {"pa_append_kv", "pa_forward", "pa_forward_workspace_bytes",
                                       "pa_last_error"}
    # the op's attributes carry no testing hook
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    for hook in ("path", "split_tokens", "prefill_pieces", "prefill_kernel"):
        assert not re.search(rf"\b{hook}\s*;", text), hook


def test_library_exports_every_declared_function():
    lib = _lib.load()
    for header, names in (("pa.h", _lib.EXPORTED), ("pa_testing.h", _lib.TESTING_EXPORTED)):
        for name in header_functions(header):
            assert hasattr(lib, name), name
        assert set(header_functions(header)) == set(names), header


def params(**kw):
    d = dict(num_heads=8, kv_num_heads=2, head_size=64, block_size=16, scale=0.0, softcap=0.0,
             local_window_size=-1, do_rotary=0, rotary_interleaved=0, cache_dtype=0,
             k_quant_type=0, v_quant_type=0,
             head_sink=None, use_smooth_softmax=0, q_norm_weight=None, k_norm_weight=None,
             qk_norm_epsilon=0.0, kv_cache_layout=0, v_head_size=0, rotary_offset=0)
    d.update(kw)
    return _lib.AttnParams(*[d[f] for f, _ in _lib.AttnParams._fields_])


def paged(**kw):
    d = dict(key_cache=FAKE, value_cache=FAKE, num_blocks=32, block_table=FAKE,
             max_blocks_per_seq=8, cumulative_sequence_length=FAKE, past_seqlens=FAKE,
             batch_size=4, token_count=4, slot_mapping=None, k_scale=None, v_scale=None)
    d.update(kw)
    return _lib.PagedKV(*[d[f] for f, _ in _lib.PagedKV._fields_])


def routing(**kw):
    d = dict(path=0, split_tokens=0, prefill_pieces=0, prefill_kernel=0)
    d.update(kw)
    return _lib.Routing(*[d[f] for f, _ in _lib.Routing._fields_])


def call_forward(p, kv, query=FAKE, cos=None, sin=None, rows=0, rdim=0, mq=0, mk=0, ws=None,
                 ws_len=0, out=FAKE, rt=None):
    lib = _lib.load()
    if rt is None:
        return lib.pa_forward(ctypes.byref(p), ctypes.byref(kv), query, cos, sin, rows, rdim, mq,
                              mk, ws, ws_len, out, None)
    return lib.pa_forward_routed(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(rt), query, cos,
                                 sin, rows, rdim, mq, mk, ws, ws_len, out, None)


def call_append(p, kv, key=FAKE, value=FAKE, cos=None, sin=None, rows=0, rdim=0):
    lib = _lib.load()
    return lib.pa_append_kv(ctypes.byref(p), ctypes.byref(kv), key, value, cos, sin, rows, rdim,
                            None)


def err():
    return _lib.load().pa_last_error().decode()


NEGATIVE = [
    # (params overrides, kv overrides, expected status, message fragment)
    (dict(num_heads=0), {}, 1, "num_heads"),
    (dict(kv_num_heads=0), {}, 1, "kv_num_heads"),
    (dict(num_heads=6, kv_num_heads=4), {}, 1, "multiple of kv_num_heads"),
    (dict(head_size=60), {}, 1, "head_size"),
    (dict(block_size=24), {}, 1, "block_size"),
    (dict(block_size=8), {}, 1, "block_size"),
    (dict(scale=float("inf")), {}, 1, "scale"),
    (dict(softcap=-1.0), {}, 1, "softcap"),
    (dict(softcap=float("nan")), {}, 1, "softcap"),
    (dict(local_window_size=0), {}, 1, "local_window_size"),
    (dict(local_window_size=-2), {}, 1, "local_window_size"),
    (dict(do_rotary=2), {}, 1, "do_rotary"),
    (dict(rotary_interleaved=3), {}, 1, "rotary_interleaved"),
    ({}, dict(batch_size=0), 1, "batch_size"),
    ({}, dict(token_count=-1), 1, "token_count"),
    ({}, dict(num_blocks=0), 1, "num_blocks"),
    ({}, dict(num_blocks=(1 << 28) + 1), 1, "2^32 slots"),
    ({}, dict(max_blocks_per_seq=0), 1, "max_blocks_per_seq"),
    ({}, dict(key_cache=None), 1, "key_cache"),
    ({}, dict(value_cache=FAKE + 8), 1, "16-byte"),
    ({}, dict(block_table=None), 1, "block_table"),
    ({}, dict(cumulative_sequence_length=None), 1, "cumulative_sequence_length"),
    ({}, dict(past_seqlens=None), 1, "past_seqlens"),
    # quantized caches (section 8.7)
    (dict(cache_dtype=3), {}, 1, "cache_dtype"),
    (dict(cache_dtype=-1), {}, 1, "cache_dtype"),
    (dict(k_quant_type=3), {}, 1, "k_quant_type"),
    (dict(v_quant_type=-1), {}, 1, "v_quant_type"),
    (dict(k_quant_type=1), dict(k_scale=FAKE), 1, "expected NONE with an fp16 cache"),
    ({}, dict(k_scale=FAKE), 1, "k_scale: given but k_quant_type is NONE"),
    ({}, dict(v_scale=FAKE), 1, "v_scale: given but v_quant_type is NONE"),
    (dict(cache_dtype=1, k_quant_type=1), dict(k_scale=FAKE), 1,
     "expected PER_TENSOR or PER_CHANNEL"),
    (dict(cache_dtype=2), {}, 1, "expected PER_TENSOR or PER_CHANNEL"),
    (dict(cache_dtype=1, k_quant_type=1, v_quant_type=2), dict(k_scale=FAKE), 1,
     "v_scale: required when v_quant_type is PER_CHANNEL"),
    (dict(cache_dtype=2, k_quant_type=2, v_quant_type=1), dict(k_scale=FAKE + 4, v_scale=FAKE),
     1, "k_scale: expected 16-byte alignment for PER_CHANNEL"),
    (dict(cache_dtype=2, k_quant_type=1, v_quant_type=1), dict(k_scale=FAKE, v_scale=FAKE + 2),
     1, "v_scale: expected 4-byte alignment"),
]

# attention sink and QK-Norm (sections 6.4, 7.4)
NEGATIVE += [
    (dict(use_smooth_softmax=2), {}, 1, "use_smooth_softmax"),
    (dict(head_sink=FAKE + 1), {}, 1, "head_sink: expected 2-byte"),
    (dict(q_norm_weight=FAKE), {}, 1, "both or neither"),
    (dict(k_norm_weight=FAKE), {}, 1, "both or neither"),
    (dict(q_norm_weight=FAKE, k_norm_weight=FAKE + 8), {}, 1, "16-byte alignment"),
    (dict(qk_norm_epsilon=-1e-6), {}, 1, "qk_norm_epsilon"),
    (dict(qk_norm_epsilon=float("inf")), {}, 1, "qk_norm_epsilon"),
]

# latent layout (MLA, section 12.10) and offset RoPE
LAT = dict(kv_cache_layout=1, kv_num_heads=1, num_heads=8, head_size=576, v_head_size=512,
           scale=0.07)
LAT_KV = dict(value_cache=None)
NEGATIVE += [
    ({}, dict(value_cache=None), 1, "value_cache: expected non-NULL"),
    (dict(kv_cache_layout=2), {}, 1, "kv_cache_layout"),
    (dict(v_head_size=-1), {}, 1, "v_head_size: expected 0..head_size"),
    (dict(v_head_size=32), {}, 1, "requires kv_cache_layout LATENT"),
    (dict(rotary_offset=4), {}, 1, "rotary_offset"),
    (dict(LAT, kv_num_heads=2), LAT_KV, 1, "kv_num_heads: expected 1"),
    (LAT, {}, 1, "value_cache: expected NULL"),
    (dict(LAT, scale=0.0), LAT_KV, 1, "explicit scale"),
    (dict(LAT, use_smooth_softmax=1), LAT_KV, 1, "not allowed with kv_cache_layout LATENT"),
    (dict(LAT, cache_dtype=1, k_quant_type=1, v_quant_type=1), dict(LAT_KV, k_scale=FAKE,
     v_scale=FAKE), 1, "v_quant_type/v_scale"),
]

QUANT = dict(cache_dtype=1, k_quant_type=1, v_quant_type=2)
QUANT_KV = dict(k_scale=FAKE + 4, v_scale=FAKE)     # per tensor: 4-byte; per channel: 16-byte


@pytest.mark.parametrize("pk,kk,status,frag", NEGATIVE)
def test_validation_rule(pk, kk, status, frag):
    for call in (call_forward, call_append):
        st = call(params(**pk), paged(**kk))
        assert st == status, (call.__name__, err())
        assert frag in err(), err()


ROUTING_NEGATIVE = [
    (dict(path=3), "path"),
    (dict(split_tokens=100), "split_tokens"),
    (dict(prefill_pieces=5), "prefill_pieces"),
    (dict(prefill_pieces=-1), "prefill_pieces"),
    (dict(prefill_kernel=4), "prefill_kernel"),
    (dict(prefill_kernel=-1), "prefill_kernel"),
]


@pytest.mark.parametrize("rk,frag", ROUTING_NEGATIVE)
def test_routing_validation_rule(rk, frag):
    lib = _lib.load()
    assert call_forward(params(), paged(), rt=routing(**rk)) == 1 and frag in err(), err()
    n = ctypes.c_size_t(0)
    r = routing(**rk)
    assert lib.pa_forward_workspace_bytes_routed(ctypes.byref(params()), ctypes.byref(paged()),
                                                 ctypes.byref(r), 0, 0, ctypes.byref(n)) == 1
    buf = ctypes.create_string_buffer(64)
    assert lib.pa_describe_plan(ctypes.byref(params()), ctypes.byref(paged()), ctypes.byref(r),
                                0, 0, buf, 64) == 1 and frag in err()


def test_stream_read_rules():
    lib = _lib.load()
    assert lib.pa_bench_stream_read(FAKE, 1000, FAKE, None) == 1 and "16384" in err()
    assert lib.pa_bench_stream_read(FAKE + 8, 16384, FAKE, None) == 1 and "src" in err()
    assert lib.pa_bench_stream_read(None, 16384, FAKE, None) == 1
    assert lib.pa_bench_stream_read(FAKE, 0, FAKE, None) == 0


def test_rotary_rules():
    kv = paged()
    p = params(do_rotary=1)
    assert call_forward(p, kv) == 1 and "required when do_rotary" in err()
    assert call_append(p, kv, cos=FAKE) == 1 and "both or neither" in err()
    assert call_forward(p, kv, cos=FAKE, sin=FAKE, rows=128, rdim=66) == 1 and "rotary_dim" in err()
    assert call_forward(p, kv, cos=FAKE, sin=FAKE, rows=128, rdim=7) == 1 and "rotary_dim" in err()
    assert call_forward(p, kv, cos=FAKE, sin=FAKE, rows=127, rdim=64) == 1 and "rotary_rows" in err()
    assert call_append(params(), kv, cos=FAKE, sin=FAKE, rows=128, rdim=64) == 1 \
        and "do_rotary = 0" in err()


def test_forward_buffer_rules():
    kv = paged()
    assert call_forward(params(), kv, query=None) == 1 and "query" in err()
    assert call_forward(params(), kv, out=None) == 1 and "out" in err()
    assert call_forward(params(), kv, query=FAKE + 2) == 1 and "16-byte" in err()
    assert call_append(params(), kv, key=None) == 1 and "key/value" in err()
    assert call_forward(params(), kv, mq=-1) == 1 and "bound" in err()


def test_slot_mapping_alignment_rule():
    assert call_append(params(), paged(slot_mapping=FAKE + 2)) == 1 and "slot_mapping" in err()


def test_unsupported_head_size_is_reported():
    assert call_forward(params(head_size=96), paged()) == 2
    assert "head_size 96" in err()


def test_rows16_prefill_kernel_limits():
    # the 8-wave prefill kernel serves head_size 256 with caches below 4 GiB
    rt = routing(prefill_kernel=2)
    assert call_forward(params(), paged(), rt=rt) == 2 and "prefill_kernel 2" in err()
    big = paged(num_blocks=(1 << 32) // (16 * 2 * 256 * 2))   # exactly 4 GiB per cache
    assert call_forward(params(head_size=256), big, rt=rt) == 2
    assert "4 GiB" in err()


def test_rows32_prefill_kernel_limits():
    # the 32-row 8-wave prefill kernel serves head_size 256 with caches below
    # 4 GiB
    rt = routing(prefill_kernel=3)
    assert call_forward(params(), paged(), rt=rt) == 2 and "prefill_kernel 3" in err()
    big = paged(num_blocks=(1 << 32) // (16 * 2 * 256 * 2))   # exactly 4 GiB per cache
    assert call_forward(params(head_size=256), big, rt=rt) == 2
    assert "4 GiB" in err()


def test_quantized_cache_routing():
    # decode rows read codes in the decode kernel; multi-token requests take
    # the prefill kernel, as with an fp16 cache (the same static shape test)
    pl = plan(params(**QUANT), paged(token_count=40, batch_size=4, **QUANT_KV))
    assert pl["mode"] == "request" and pl["cache"] == "int8" and pl["prefill_grid"] != "(0,0)"
    pl = plan(params(cache_dtype=2, k_quant_type=2, v_quant_type=2),
              paged(token_count=4, batch_size=4, k_scale=FAKE, v_scale=FAKE))
    assert pl["mode"] == "token" and pl["cache"] == "fp8e4m3fn"
    assert plan(params(), paged())["cache"] == "fp16"
    # forced routes: every token on the decode kernel, or the prefill kernel
    pl = plan(params(**QUANT), paged(token_count=40, batch_size=4, **QUANT_KV), rt=routing(path=1))
    assert pl["mode"] == "token" and pl["prefill_grid"] == "(0,0)"
    pl = plan(params(**QUANT), paged(token_count=4, batch_size=4, **QUANT_KV), rt=routing(path=2))
    assert pl["mode"] == "request"
    # every prefill kernel reads codes, the 16-row 8-wave one included
    pl = plan(params(head_size=256, **QUANT), paged(token_count=40, batch_size=4, **QUANT_KV),
              rt=routing(prefill_kernel=2))
    assert pl["mode"] == "request" and pl["cache"] == "int8"


def test_qk_norm_head_size_limit_and_workspace():
    norm = dict(q_norm_weight=FAKE, k_norm_weight=FAKE)
    assert call_forward(params(head_size=96, **norm), paged()) == 2
    assert call_append(params(head_size=96, **norm), paged()) == 2 and "QK-Norm" in err()
    # the normalized queries are staged in the workspace: T * H * D fp16
    a = plan(params(), paged(token_count=4, batch_size=4))
    b = plan(params(**norm), paged(token_count=4, batch_size=4))
    assert b["q_norm"] == "1" and a["q_norm"] == "0"
    assert int(b["workspace"]) - int(a["workspace"]) >= 4 * 8 * 64 * 2


def test_latent_rules():
    kv = paged(**LAT_KV)
    # RoPE must leave the V channels (the leading 512) alone
    p = params(**LAT, do_rotary=1, rotary_offset=256)
    assert call_forward(p, kv, cos=FAKE, sin=FAKE, rows=128, rdim=64) == 1
    assert "rotary_offset" in err()
    # offset + rotary_dim within the head
    p = params(**LAT, do_rotary=1, rotary_offset=544)
    assert call_forward(p, kv, cos=FAKE, sin=FAKE, rows=128, rdim=64) == 1
    assert "rotary_dim" in err()
    # the append takes no value rows
    assert call_append(params(**LAT), kv) == 1 and "value: expected NULL" in err()
    # kernel shapes: 576/512 fp16 only; path 2 has no latent kernel
    assert call_forward(params(**dict(LAT, head_size=64, v_head_size=32)), kv) == 2
    assert "LATENT: served for head_size 576" in err()
    assert call_forward(params(**LAT), kv, rt=routing(path=2)) == 2 and "latent kernel" in err()
    big = paged(value_cache=None, num_blocks=(1 << 32) // (16 * 576 * 2) + 1)
    assert call_forward(params(**LAT), big) == 2 and "4 GiB" in err()
    pl = plan(params(**LAT), paged(token_count=40, batch_size=4, **LAT_KV))
    assert pl["mode"] == "token" and pl["prefill_grid"] == "(0,0)"


def test_workspace_must_cover_the_plan():
    lib = _lib.load()
    p, kv = params(), paged(token_count=64, batch_size=64, max_blocks_per_seq=1024)
    n = ctypes.c_size_t(0)
    assert lib.pa_forward_workspace_bytes(ctypes.byref(p), ctypes.byref(kv), 0, 0,
                                          ctypes.byref(n)) == 0
    assert n.value > 0
    assert call_forward(p, kv, ws=FAKE, ws_len=n.value - 1) == 1 and "workspace_bytes" in err()
    assert call_forward(p, kv, ws=None, ws_len=n.value) == 1 and "workspace" in err()


def test_zero_tokens_is_a_no_op():
    kv = paged(token_count=0)
    assert call_forward(params(), kv, query=None, out=None) == 0
    assert call_append(params(), kv, key=None, value=None) == 0


def plan(p, kv, mq=0, mk=0, rt=None):
    lib = _lib.load()
    buf = ctypes.create_string_buffer(512)
    r = None if rt is None else ctypes.byref(rt)
    assert lib.pa_describe_plan(ctypes.byref(p), ctypes.byref(kv), r, mq, mk, buf, 512) == 0, err()
    return dict(kv.split("=", 1) for kv in buf.value.decode().split())


def test_plan_static_shape_test():
    """token_count <= batch_size selects the decode kernel for every token;
    otherwise requests of one token go to decode and the rest to prefill."""
    assert plan(params(), paged(token_count=4, batch_size=4))["mode"] == "token"
    pl = plan(params(), paged(token_count=40, batch_size=4))
    assert pl["mode"] == "request" and pl["prefill_grid"] != "(0,0)"
    assert plan(params(), paged(token_count=40, batch_size=4), rt=routing(path=1))["mode"] == "token"
    assert plan(params(), paged(token_count=4, batch_size=4), rt=routing(path=2))["mode"] == "request"


def test_plan_split_length_ignores_bounds():
    """Bounds only trim the grid and workspace: the split length (and so the
    arithmetic of every row) is the same with no, tight or loose bounds."""
    p, kv = params(), paged(token_count=8, batch_size=8, max_blocks_per_seq=512)
    a, b, c = plan(p, kv), plan(p, kv, 1, 3000), plan(p, kv, 10 ** 6, 10 ** 8)
    assert a["split_tokens"] == b["split_tokens"] == c["split_tokens"]
    assert int(b["max_splits"]) <= int(a["max_splits"]) == int(c["max_splits"])


def test_plan_window_caps_splits():
    p = params(local_window_size=100)
    pl = plan(p, paged(token_count=2, batch_size=2, max_blocks_per_seq=4096))
    assert int(pl["max_splits"]) * int(pl["split_tokens"]) < 100 + int(pl["split_tokens"])


def test_plan_group_chunks():
    pl = plan(params(num_heads=24, kv_num_heads=2), paged())      # g = 12: one chunk
    assert pl["g"] == "12" and pl["chunk_heads"] == "12" and pl["head_chunks"] == "2"
    pl = plan(params(num_heads=64, kv_num_heads=2), paged())      # g = 32: chunks of 16
    assert pl["chunk_heads"] == "16" and pl["head_chunks"] == "4"
    pl = plan(params(num_heads=40, kv_num_heads=2), paged())      # g = 20: chunks of 10
    assert pl["chunk_heads"] == "10"


def test_noalloc_rejects_a_plan_beyond_its_scratch_before_any_device_call():
    lib = _lib.load()
    p = params(num_heads=64, kv_num_heads=8, head_size=256)
    kv = paged(token_count=64, batch_size=64, max_blocks_per_seq=8192, num_blocks=1 << 16)
    assert int(plan(p, kv)["workspace"]) > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.pa_forward_noalloc(ctypes.byref(p), ctypes.byref(kv), FAKE, None, None, 0, 0, 0, 0,
                                FAKE, None)
    assert st == 2 and "scratch array" in err(), err()
    # validation runs first, as for pa_forward
    st = lib.pa_forward_noalloc(ctypes.byref(params(num_heads=0)), ctypes.byref(paged()), FAKE,
                                None, None, 0, 0, 0, 0, FAKE, None)
    assert st == 1 and "num_heads" in err()
    assert lib.pa_forward_noalloc(ctypes.byref(params()), ctypes.byref(paged(token_count=0)),
                                  None, None, None, 0, 0, 0, 0, None, None) == 0
