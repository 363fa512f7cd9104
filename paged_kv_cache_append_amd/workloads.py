"""Seeded synthetic inputs for paged KV append + PagedAttention forward.

This module only *draws* inputs: lengths, block tables, new Q/K/V tokens,
block-pool contents and rotary tables.  It holds none of the attention
arithmetic, so that both the fp64 oracle (``oracle/``) and the HIP path can
consume the very same host arrays without sharing any code of the method.

Input contract being populated (PagedAttention -- CUDA Design Document, §4 and
§4.3; Design: WebGPU PagedAttention, §3.3 "GenAI runtime contract"):

* ``query``  fp16 ``[token_count, num_heads * head_size]`` packed over requests
* ``key``/``value`` fp16 ``[token_count, kv_num_heads * head_size]``
* ``key_cache``/``value_cache`` fp16 ``[num_blocks, block_size, kv_num_heads, head_size]``
* ``block_table`` int32 ``[batch_size, max_blocks_per_seq]`` (entry i holds the
  block of positions ``[i*block_size, (i+1)*block_size)``; padding is -1)
* ``cumulative_sequence_lengths`` int32 ``[batch_size + 1]``
* ``past_sequence_lengths`` int32 ``[batch_size]``
* ``cos_cache``/``sin_cache`` fp16 ``[rows, rotary_dim / 2]`` when rotary is on.

Pool contents are generated per physical block from a counter-keyed numpy
generator ``default_rng([seed, kind, block])`` so any subset of blocks can be
re-drawn without materialising the whole pool (the 256-sequence decode pool is
about 10 GB).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

KIND_K = 0
KIND_V = 1


@dataclass
class Workload:
    """One batch of synthetic inputs for an append + forward step."""

    name: str
    seed: int
    num_heads: int
    kv_num_heads: int
    head_size: int
    block_size: int
    scale: float
    softcap: float
    local_window_size: int
    do_rotary: int
    rotary_interleaved: int
    cum: np.ndarray            # int32 [B+1]
    past: np.ndarray           # int32 [B]
    block_table: np.ndarray    # int32 [B, max_blocks_per_seq]
    num_blocks: int
    query: np.ndarray          # fp16 [T, H*D]
    key: np.ndarray            # fp16 [T, Hkv*D]
    value: np.ndarray          # fp16 [T, Hkv*D]
    cos_cache: Optional[np.ndarray] = None   # fp16 [rows, rot/2]
    sin_cache: Optional[np.ndarray] = None
    kv_sigma: float = 1.0
    # blocks whose contents are NaN before the append ("poisoned" pool):
    # every slot that the runtime has not filled yet.
    poison: bool = False
    description: str = ""
    extra: dict = field(default_factory=dict)

    # ---- shape helpers -------------------------------------------------
    @property
    def batch_size(self) -> int:
        return int(self.past.shape[0])

    @property
    def token_count(self) -> int:
        return int(self.query.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cum.astype(np.int64))

    @property
    def rotary_dim(self) -> int:
        return 0 if self.cos_cache is None else 2 * int(self.cos_cache.shape[1])

    @property
    def rotary_rows(self) -> int:
        return 0 if self.cos_cache is None else int(self.cos_cache.shape[0])

    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.kv_num_heads, self.head_size)

    # ---- pool contents -------------------------------------------------
    def pool_blocks(self, kind: int, ids: Sequence[int]) -> np.ndarray:
        """fp16 contents of physical blocks ``ids`` of the K (kind 0) or V
        (kind 1) pool, before the append."""
        ids = [int(i) for i in ids]
        out = np.empty((len(ids), self.block_size, self.kv_num_heads, self.head_size),
                       np.float16)
        for n, p in enumerate(ids):
            out[n] = _draw_block(self.seed, kind, p, out.shape[1:], self.kv_sigma)
        dead = self.extra.get("dead_blocks")
        if dead:
            for n, p in enumerate(ids):
                if p in dead:
                    out[n] = np.float16(np.nan)
        if self.poison:
            filled = self._filled_tokens()
            for n, p in enumerate(ids):
                f = filled.get(p, 0)
                out[n, f:] = np.float16(np.nan)
        return out

    def code_blocks(self, kind: int, ids: Sequence[int], cache_dtype: int) -> np.ndarray:
        """Codes of physical blocks ``ids`` of a quantized K (kind 0) or V
        (kind 1) pool, before the append."""
        ids = [int(i) for i in ids]
        shape = (self.block_size, self.kv_num_heads, self.head_size)
        out = np.empty((len(ids),) + shape, code_dtype(cache_dtype))
        for n, p in enumerate(ids):
            out[n] = draw_code_block(self.seed, kind, p, shape, cache_dtype)
        dead = self.extra.get("dead_blocks")
        if dead:
            # int8 has no NaN: the largest code, which a wrong read would show
            for n, p in enumerate(ids):
                if p in dead:
                    out[n] = 0x7F
        if self.poison and cache_dtype == CACHE_FP8:
            # unfilled slots hold the e4m3fn NaN code (int8 has no NaN)
            filled = self._filled_tokens()
            for n, p in enumerate(ids):
                out[n, filled.get(p, 0):] = 0x7F
        return out

    def full_pool(self, kind: int, threads: Optional[int] = None,
                  chunk: int = 512) -> np.ndarray:
        """The whole pool of one kind, drawn block by block (threaded)."""
        pool = np.empty(self.pool_shape(), np.float16)
        fill_pool_chunks(self, kind, pool, threads=threads, chunk=chunk)
        return pool

    def _filled_tokens(self) -> dict:
        """Physical block -> number of leading slots that hold cached tokens
        (the runtime's bookkeeping of what it has written so far)."""
        if "_filled" in self.extra:
            return self.extra["_filled"]
        filled = {}
        bs = self.block_size
        for b in range(self.batch_size):
            n_past = int(self.past[b])
            for i in range(self.max_blocks_per_seq):
                blk = int(self.block_table[b, i])
                if blk < 0:
                    continue
                n = min(max(n_past - i * bs, 0), bs)
                filled[blk] = max(filled.get(blk, 0), n)
        self.extra["_filled"] = filled
        return filled


def _draw_block(seed: int, kind: int, p: int, shape, sigma: float) -> np.ndarray:
    rng = np.random.default_rng([seed, kind, p])
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x.astype(np.float16)


def fill_pool_chunks(w: Workload, kind: int, out: np.ndarray,
                     threads: Optional[int] = None, chunk: int = 512,
                     sink=None) -> None:
    """Draw every block of one pool kind into ``out`` (host array).  If
    ``sink`` is given it is called as ``sink(start, array)`` per chunk (used to
    stream the pool to device memory without holding it all on the host)."""
    fill_chunks(w, kind, out, lambda ids: w.pool_blocks(kind, ids), threads, chunk, sink)


def fill_chunks(w: Workload, kind: int, out, draw, threads: Optional[int] = None,
                chunk: int = 512, sink=None) -> None:
    """Run ``draw(block ids)`` over the pool in chunks (threaded), writing
    into ``out`` and/or handing each chunk to ``sink(start, array)``."""
    nb = w.num_blocks
    threads = threads or min(16, os.cpu_count() or 1)

    def work(start):
        stop = min(nb, start + chunk)
        arr = draw(range(start, stop))
        return start, arr

    with ThreadPoolExecutor(threads) as ex:
        for start, arr in ex.map(work, range(0, nb, chunk)):
            if out is not None:
                out[start:start + arr.shape[0]] = arr
            if sink is not None:
                sink(start, arr)


# ---------------------------------------------------------------------------
# quantized caches: byte codes of the pool and fp32 scales (drawn, never
# computed from fp16 values -- the quantizer lives on each side separately)
# ---------------------------------------------------------------------------

CACHE_FP16, CACHE_INT8, CACHE_FP8 = 0, 1, 2
QUANT_NONE, QUANT_PER_TENSOR, QUANT_PER_CHANNEL = 0, 1, 2


def code_dtype(cache_dtype: int):
    """numpy dtype of a quantized pool: int8 codes, or e4m3fn bytes as uint8."""
    return np.int8 if cache_dtype == CACHE_INT8 else np.uint8


def draw_code_block(seed: int, kind: int, p: int, shape, cache_dtype: int) -> np.ndarray:
    """Codes of one physical block of a quantized pool.  int8: a rounded
    normal of standard deviation 36 clipped to the int8 range (a tail of
    saturated codes included).  e4m3fn: random sign, exponent field drawn
    around 12.5 with deviation 0.8 (values of about 2^6, tails comparable to a
    normal's), random mantissa; the NaN bytes 0x7f and 0xff are replaced by
    the largest finite codes."""
    rng = np.random.default_rng([seed, kind, p, 100 + cache_dtype])
    if cache_dtype == CACHE_INT8:
        x = np.rint(rng.standard_normal(shape) * 36.0)
        return np.clip(x, -128, 127).astype(np.int8)
    e = np.clip(np.rint(rng.normal(12.5, 0.8, shape)), 0, 15).astype(np.uint8)
    m = rng.integers(0, 8, shape, dtype=np.uint8)
    s = rng.integers(0, 2, shape, dtype=np.uint8)
    c = (s << 7) | (e << 3) | m
    c[(c & 0x7F) == 0x7F] -= 1
    return c.astype(np.uint8)


def draw_scales(w: "Workload", kind: int, cache_dtype: int, quant_type: int,
                seed: int) -> np.ndarray:
    """fp32 scales of one quantized cache: ``[1]`` (per tensor) or
    ``[Hkv, D]`` (per channel).  The base puts the new tokens' values
    (standard deviation ``kv_sigma``) at about 36 int8 steps (so about one in
    300 saturates) or about 2^6.3 on the e4m3fn grid; per-channel scales
    spread the base by a factor drawn from [2^-0.5, 2^0.5)."""
    rng = np.random.default_rng([seed, kind, 200 + cache_dtype, quant_type])
    base = w.kv_sigma / 36.0 if cache_dtype == CACHE_INT8 else w.kv_sigma / 80.0
    if quant_type == QUANT_PER_TENSOR:
        return np.array([base * rng.uniform(0.8, 1.25)], np.float32)
    f = 2.0 ** rng.uniform(-0.5, 0.5, (w.kv_num_heads, w.head_size))
    return (base * f).astype(np.float32)


def rope_tables(rows: int, rotary_dim: int, base: float = 10000.0):
    """fp16 cos/sin tables ``[rows, rotary_dim/2]`` for the standard inverse
    frequency ``base**(-2i/rotary_dim)``, evaluated in fp64 then rounded."""
    half = rotary_dim // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / rotary_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float16), np.sin(ang).astype(np.float16)


def build_case(name: str, seed: int, *, q_lens: Sequence[int], past: Sequence[int],
               num_heads: int, kv_num_heads: int, head_size: int, block_size: int,
               scale: float = 0.0, softcap: float = 0.0, local_window_size: int = -1,
               do_rotary: int = 0, rotary_interleaved: int = 0, rotary_dim: int = 0,
               rotary_base: float = 10000.0, q_sigma: float = 1.0, kv_sigma: float = 1.0,
               num_blocks: Optional[int] = None, pool_slack: float = 1.1,
               extra_blocks_per_seq: int = 0, rng: Optional[np.random.Generator] = None,
               shuffle: bool = True, poison: bool = False, description: str = "",
               extra_tokens: int = 0) -> Workload:
    """Assemble a workload from explicit per-sequence lengths.

    Block allocation mimics a serving runtime: each sequence gets
    ``ceil((past + q_len) / block_size)`` physical blocks taken in batch order
    from a seeded permutation of the pool; unused table entries are -1.
    ``extra_tokens`` appends rows to the packed Q/K/V beyond the last
    sequence (tokens owned by no sequence)."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    past = np.asarray(past, dtype=np.int64)
    B = len(q_lens)
    assert len(past) == B
    kv_lens = past + q_lens
    nblk = (kv_lens + block_size - 1) // block_size
    used = int(nblk.sum())
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_slack * used)))
    assert num_blocks >= used, "pool too small"
    maxblk = max(1, int(nblk.max()) + extra_blocks_per_seq) if B else 1
    perm = rng.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    table = np.full((B, maxblk), -1, np.int32)
    o = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = perm[o:o + n]
        o += n
    cum = np.zeros(B + 1, np.int32)
    cum[1:] = np.cumsum(q_lens)
    T = int(cum[-1]) + extra_tokens
    H, Hkv, D = num_heads, kv_num_heads, head_size
    q = rng.standard_normal((T, H * D), dtype=np.float32)
    if q_sigma != 1.0:
        q *= np.float32(q_sigma)
    k = rng.standard_normal((T, Hkv * D), dtype=np.float32) * np.float32(kv_sigma)
    v = rng.standard_normal((T, Hkv * D), dtype=np.float32) * np.float32(kv_sigma)
    cos = sin = None
    if do_rotary:
        rd = rotary_dim or D
        rows = maxblk * block_size
        cos, sin = rope_tables(rows, rd, rotary_base)
    w = Workload(name=name, seed=seed, num_heads=H, kv_num_heads=Hkv, head_size=D,
                 block_size=block_size, scale=float(scale), softcap=float(softcap),
                 local_window_size=int(local_window_size), do_rotary=int(do_rotary),
                 rotary_interleaved=int(rotary_interleaved), cum=cum,
                 past=past.astype(np.int32), block_table=table, num_blocks=int(num_blocks),
                 query=q.astype(np.float16), key=k.astype(np.float16),
                 value=v.astype(np.float16), cos_cache=cos, sin_cache=sin,
                 kv_sigma=float(kv_sigma), poison=poison, description=description)
    w.extra["perm"] = perm
    return w


# ---------------------------------------------------------------------------
# The five benchmark workloads C1..C5 (seed 1000 + n for config Cn, draws in a
# fixed order: past lengths, block permutation, Q, K, V; pool per block).
# ---------------------------------------------------------------------------

CONFIG_NAMES = (
    "tiny_decode",
    "llama3_8b_mixed",
    "decode_heavy_256",
    "gemma2_prefill_window",
    "long_context_decode_rope",
)


def make_workload(name: str, poison: bool = False) -> Workload:
    idx = CONFIG_NAMES.index(name)
    seed = 1001 + idx
    rng = np.random.default_rng(seed)
    if name == "tiny_decode":
        # 2 sequences, one new token each on 37 / 50 cached tokens; pool of 16
        # blocks; the table rows are the config's own block permutation
        # reshaped to [2, 8] (all 8 entries valid, 3 and 4 of them in use).
        w = build_case(name, seed, q_lens=[1, 1], past=[37, 50], num_heads=4,
                       kv_num_heads=2, head_size=64, block_size=16, scale=0.125,
                       num_blocks=16, rng=rng, shuffle=True, poison=poison,
                       description="2 seqs x 1 token, past 37/50, H=4 Hkv=2 D=64 bs=16")
        w.block_table = w.extra["perm"].astype(np.int32).reshape(2, 8)
        w.extra.pop("_filled", None)
        return w
    if name == "llama3_8b_mixed":
        past_dec = rng.integers(128, 4096, size=64, endpoint=True)
        q_lens = [1] * 64 + [512, 512]
        past = list(past_dec) + [0, 1024]
        return build_case(name, seed, q_lens=q_lens, past=past, num_heads=32, kv_num_heads=8,
                          head_size=128, block_size=16, scale=1.0 / math.sqrt(128), rng=rng,
                          poison=poison,
                          description="64 decode seqs (past U[128,4096]) + 2x512-token "
                                      "prefill chunks (past 0, 1024); H=32 Hkv=8 D=128 bs=16")
    if name == "decode_heavy_256":
        past = rng.integers(1024, 16384, size=256, endpoint=True)
        return build_case(name, seed, q_lens=[1] * 256, past=past, num_heads=32,
                          kv_num_heads=8, head_size=128, block_size=32,
                          scale=1.0 / math.sqrt(128), kv_sigma=0.5, rng=rng, poison=poison,
                          description="256 decode seqs, past U[1024,16384]; H=32 Hkv=8 "
                                      "D=128 bs=32; K/V ~ N(0, 0.5)")
    if name == "gemma2_prefill_window":
        return build_case(name, seed, q_lens=[2048] * 8, past=[2048] * 8, num_heads=16,
                          kv_num_heads=8, head_size=256, block_size=16, scale=1.0 / 16.0,
                          softcap=50.0, local_window_size=4096, rng=rng, poison=poison,
                          description="8 seqs x 2048 new tokens on 2048 cached; H=16 Hkv=8 "
                                      "D=256 bs=16; window 4096, softcap 50")
    if name == "long_context_decode_rope":
        past_small = rng.integers(512, 8192, size=7, endpoint=True)
        past = [131072] + list(past_small)
        return build_case(name, seed, q_lens=[1] * 8, past=past, num_heads=64, kv_num_heads=8,
                          head_size=64, block_size=64, scale=0.125, do_rotary=1,
                          rotary_interleaved=0, rotary_dim=64, rng=rng, poison=poison,
                          description="1 seq on 131072 cached + 7 on U[512,8192]; H=64 "
                                      "Hkv=8 D=64 bs=64; rotary base 10000")
    raise KeyError(name)


# ---------------------------------------------------------------------------
# Latent attention (MLA) workloads: absorbed DeepSeek-style rows of 576
# channels (512 latent + 64 rotary at offset 512), one kv head, V = the
# leading 512 channels (PagedAttention -- CUDA Design Document, section 12).
# The scale is 1/sqrt(192), the pre-absorption head width (section 12.6).
# seed 1100 + index; extra["latent"] marks them (value rows are drawn but
# unused).
# ---------------------------------------------------------------------------

MLA_CONFIG_NAMES = ("mla_decode_tp8", "mla_decode_dp")
MLA_HEAD_SIZE, MLA_V_HEAD_SIZE, MLA_ROTARY_OFFSET, MLA_ROTARY_DIM = 576, 512, 512, 64
MLA_SCALE = 1.0 / math.sqrt(192.0)


def _mla_case(name, seed, q_lens, past, num_heads, rng, block_size=64, **kw):
    w = build_case(name, seed, q_lens=q_lens, past=past, num_heads=num_heads, kv_num_heads=1,
                   head_size=MLA_HEAD_SIZE, block_size=block_size, scale=MLA_SCALE,
                   do_rotary=1, rotary_dim=MLA_ROTARY_DIM, rng=rng, **kw)
    w.extra["latent"] = True
    w.extra["v_head_size"] = MLA_V_HEAD_SIZE
    w.extra["rotary_offset"] = MLA_ROTARY_OFFSET
    return w


def make_mla_workload(name: str) -> Workload:
    idx = MLA_CONFIG_NAMES.index(name)
    seed = 1100 + idx
    rng = np.random.default_rng(seed)
    if name == "mla_decode_tp8":
        past = rng.integers(1024, 16384, size=128, endpoint=True)
        return _mla_case(name, seed, [1] * 128, past, 16, rng,
                         description="128 decode seqs, past U[1024,16384]; H=16 (one GPU's "
                                     "share of 128 heads), latent 576/512, bs=64")
    past = rng.integers(1024, 8192, size=64, endpoint=True)
    return _mla_case(name, seed, [1] * 64, past, 128, rng,
                     description="64 decode seqs, past U[1024,8192]; H=128, latent 576/512, "
                                 "bs=64")


def scaled_down_mla(name: str) -> Workload:
    """Small stand-ins for the MLA workloads (the oracle takes seconds)."""
    idx = MLA_CONFIG_NAMES.index(name)
    seed = 2100 + idx
    rng = np.random.default_rng(seed)
    if name == "mla_decode_tp8":
        past = list(rng.integers(1, 900, size=5, endpoint=True))
        return _mla_case(name + "_small", seed, [1] * 5, past, 16, rng)
    past = list(rng.integers(1, 600, size=3, endpoint=True))
    return _mla_case(name + "_small", seed, [1] * 3, past, 128, rng)


def scaled_down(name: str, poison: bool = False) -> Workload:
    """A small stand-in with the same head layout, block size and features as
    benchmark workload ``name`` (lengths cut so the oracle finishes in
    seconds while still spanning several tiles and a ragged tail)."""
    idx = CONFIG_NAMES.index(name)
    seed = 2000 + idx
    rng = np.random.default_rng(seed)
    if name == "tiny_decode":
        return make_workload(name, poison)
    if name == "llama3_8b_mixed":
        past = list(rng.integers(1, 700, size=6, endpoint=True)) + [0, 75]
        return build_case(name + "_small", seed, q_lens=[1] * 6 + [130, 77], past=past,
                          num_heads=32, kv_num_heads=8, head_size=128, block_size=16,
                          scale=1.0 / math.sqrt(128), rng=rng, poison=poison)
    if name == "decode_heavy_256":
        past = rng.integers(1, 1500, size=12, endpoint=True)
        return build_case(name + "_small", seed, q_lens=[1] * 12, past=past, num_heads=32,
                          kv_num_heads=8, head_size=128, block_size=32,
                          scale=1.0 / math.sqrt(128), kv_sigma=0.5, rng=rng, poison=poison)
    if name == "gemma2_prefill_window":
        return build_case(name + "_small", seed, q_lens=[150, 67], past=[200, 0], num_heads=16,
                          kv_num_heads=8, head_size=256, block_size=16, scale=1.0 / 16.0,
                          softcap=50.0, local_window_size=96, rng=rng, poison=poison)
    if name == "long_context_decode_rope":
        past = [3000] + list(rng.integers(10, 400, size=3, endpoint=True))
        return build_case(name + "_small", seed, q_lens=[1] * 4, past=past, num_heads=64,
                          kv_num_heads=8, head_size=64, block_size=64, scale=0.125,
                          do_rotary=1, rotary_interleaved=0, rotary_dim=64, rng=rng,
                          poison=poison)
    raise KeyError(name)


# ---------------------------------------------------------------------------
# device upload (PyTorch is only the memory allocator here)
# ---------------------------------------------------------------------------

def random_slot_mapping(w: Workload, seed: int, skip_fraction: float = 0.0) -> np.ndarray:
    """An explicit write-slot assignment for every token of ``w`` (int32
    ``[T]``), drawn the way a scheduler that owns placement might hand it
    out: distinct slots anywhere in the pool, each a flat index ``block *
    block_size + offset``, with about ``skip_fraction`` of the tokens given
    ``-1`` (not written: a prefix-cache hit or a rejected draft token)."""
    rng = np.random.default_rng(seed)
    n_slots = w.num_blocks * w.block_size
    T = w.token_count
    if T > n_slots:
        raise ValueError("more tokens than pool slots")
    slots = rng.choice(n_slots, size=T, replace=False).astype(np.int64)
    skip = rng.random(T) < skip_fraction
    slots[skip] = -1
    return slots.astype(np.int32)


def to_device(w: Workload, device="cuda", pools: bool = True, threads: Optional[int] = None,
              cache_dtype: int = CACHE_FP16):
    """Copy a workload's host arrays to device tensors.  Pools are streamed
    chunk by chunk so the host never holds a whole pool.  With a quantized
    ``cache_dtype`` the pools hold drawn codes (int8, or e4m3fn bytes as
    uint8)."""
    import torch
    d = {
        "query": torch.from_numpy(w.query).to(device),
        "key": torch.from_numpy(w.key).to(device),
        "value": torch.from_numpy(w.value).to(device),
        "cum": torch.from_numpy(w.cum).to(device),
        "past": torch.from_numpy(w.past).to(device),
        "block_table": torch.from_numpy(np.ascontiguousarray(w.block_table)).to(device),
        "cos": None,
        "sin": None,
    }
    if w.cos_cache is not None:
        d["cos"] = torch.from_numpy(w.cos_cache).to(device)
        d["sin"] = torch.from_numpy(w.sin_cache).to(device)
    if pools:
        tdt = {CACHE_FP16: torch.float16, CACHE_INT8: torch.int8}.get(cache_dtype, torch.uint8)
        kinds = ((KIND_K, "key_cache"),) if w.extra.get("latent") else \
            ((KIND_K, "key_cache"), (KIND_V, "value_cache"))
        d["value_cache"] = None          # a latent workload has one cache
        for kind, name in kinds:
            dev = torch.empty(w.pool_shape(), dtype=tdt, device=device)

            def sink(start, arr, dev=dev):
                dev[start:start + arr.shape[0]].copy_(torch.from_numpy(arr))

            if cache_dtype == CACHE_FP16:
                fill_pool_chunks(w, kind, None, threads=threads, sink=sink)
            else:
                fill_chunks(w, kind, None, lambda ids, k=kind: w.code_blocks(k, ids, cache_dtype),
                            threads=threads, sink=sink)
            d[name] = dev
    return d


def subset(w: Workload, seqs: Sequence[int]) -> Workload:
    """A workload holding only requests ``seqs`` of ``w`` with their blocks
    renumbered into a compact pool (contents re-drawn from ``w``'s generator,
    so they are identical).  Used to run the oracle on a sample of a large
    workload."""
    seqs = [int(s) for s in seqs]
    ids = sorted({int(x) for s in seqs for x in w.block_table[s] if x >= 0})
    remap = {old: new for new, old in enumerate(ids)}
    table = np.full((len(seqs), w.max_blocks_per_seq), -1, np.int32)
    for r, s in enumerate(seqs):
        for i, x in enumerate(w.block_table[s]):
            if x >= 0:
                table[r, i] = remap[int(x)]
    q_lens = w.q_lens[seqs]
    cum = np.zeros(len(seqs) + 1, np.int32)
    cum[1:] = np.cumsum(q_lens)
    rows = np.concatenate([np.arange(w.cum[s], w.cum[s + 1]) for s in seqs]) if len(seqs) else \
        np.zeros(0, np.int64)
    sub = Workload(name=w.name + "_subset", seed=w.seed, num_heads=w.num_heads,
                   kv_num_heads=w.kv_num_heads, head_size=w.head_size, block_size=w.block_size,
                   scale=w.scale, softcap=w.softcap, local_window_size=w.local_window_size,
                   do_rotary=w.do_rotary, rotary_interleaved=w.rotary_interleaved, cum=cum,
                   past=w.past[seqs].copy(), block_table=table, num_blocks=max(1, len(ids)),
                   query=w.query[rows], key=w.key[rows], value=w.value[rows],
                   cos_cache=w.cos_cache, sin_cache=w.sin_cache, kv_sigma=w.kv_sigma,
                   poison=w.poison)
    parent = w

    def pool_blocks(kind, bid, _ids=ids, _p=parent):
        return _p.pool_blocks(kind, [_ids[i] for i in bid])

    def code_blocks(kind, bid, cache_dtype, _ids=ids, _p=parent):
        return _p.code_blocks(kind, [_ids[i] for i in bid], cache_dtype)

    sub.pool_blocks = pool_blocks
    sub.code_blocks = code_blocks
    sub.extra["parent_rows"] = rows
    sub.extra["parent_block_ids"] = ids
    return sub


# ---------------------------------------------------------------------------
# Unmapped blocks, shared prefixes and a rolling sliding-window cache: inputs
# a serving runtime hands the op (PagedAttention -- CUDA Design Document,
# §9.2 item 3: -1 in block_table is "not mapped, masked out"; §9.3: the
# bounded-capacity window cache; §17.2: the paging tests).  Table and slot
# bookkeeping only; no attention arithmetic.
# ---------------------------------------------------------------------------

def _copy_with_table(w: Workload, table: np.ndarray, dead) -> Workload:
    import dataclasses
    extra = {k: v for k, v in w.extra.items() if k != "_filled"}
    extra["dead_blocks"] = frozenset(int(x) for x in dead) | w.extra.get("dead_blocks",
                                                                         frozenset())
    return dataclasses.replace(w, block_table=np.ascontiguousarray(table, np.int32), extra=extra)


def cached_block_entries(w: Workload):
    """(request, block index) pairs of blocks that hold only cached positions
    (no new token of this step is written there)."""
    out = []
    bs = w.block_size
    for b in range(w.batch_size):
        past = int(w.past[b])
        for i in range(past // bs):
            if int(w.block_table[b, i]) >= 0:
                out.append((b, i))
    return out


def with_unmapped_blocks(w: Workload, entries) -> Workload:
    """A copy of ``w`` whose table entries ``(request, block index)`` in
    ``entries`` are -1.  The physical blocks they named become dead: their
    contents are NaN (fp16) or the code 0x7F, so a read through a stale entry
    would show in the output."""
    table = w.block_table.copy()
    dead = set()
    for b, i in entries:
        blk = int(table[b, i])
        if blk >= 0:
            dead.add(blk)
        table[b, i] = -1
    still = {int(x) for x in table.reshape(-1) if x >= 0}
    return _copy_with_table(w, table, dead - still)


def random_unmapped_entries(w: Workload, seed: int, fraction: float):
    """About ``fraction`` of the fully cached blocks of each request, drawn."""
    rng = np.random.default_rng(seed)
    ent = cached_block_entries(w)
    keep = rng.random(len(ent)) < fraction
    return [e for e, k in zip(ent, keep) if k]


def with_shared_prefix(w: Workload, pairs) -> Workload:
    """A copy of ``w`` in which, for each ``(b1, b2, n)``, request ``b2``
    reads its first ``n`` blocks from request ``b1``'s blocks (prefix
    sharing: the blocks are read by both, written by neither; ``n`` blocks
    must hold only cached positions of both requests).  ``b2``'s former
    blocks become dead (poisoned)."""
    table = w.block_table.copy()
    bs = w.block_size
    dead = set()
    for b1, b2, n in pairs:
        if n * bs > min(int(w.past[b1]), int(w.past[b2])):
            raise ValueError("shared blocks must hold only cached positions of both requests")
        for i in range(n):
            dead.add(int(table[b2, i]))
            table[b2, i] = table[b1, i]
    still = {int(x) for x in table.reshape(-1) if x >= 0}
    return _copy_with_table(w, table, dead - still)


class RingBlockAllocator:
    """The ring-buffer policy of the bounded sliding-window cache (CUDA
    Design Document, §9.3.2 item 1): request ``b`` owns a ring of
    ``N = ceil(W / block_size) + 1`` physical blocks; position ``p`` of block
    index ``i = p // block_size`` is written to slot
    ``ring[i % N] * block_size + p % block_size`` through ``slot_mapping``,
    ``block_table[b][i]`` names ``ring[i % N]``, and entries below the window
    start of the step's earliest query are -1 (§9.3.1: the row stays indexed by
    absolute position).  Raises if a step would overwrite a block that a query
    of the same step can still see."""

    def __init__(self, batch: int, window: int, block_size: int, max_blocks_per_seq: int,
                 seed: int = 0):
        self.W, self.bs = int(window), int(block_size)
        self.N = -(-self.W // self.bs) + 1
        perm = np.random.default_rng(seed).permutation(batch * self.N)
        self.ring = perm.reshape(batch, self.N).astype(np.int32)
        self.num_blocks = batch * self.N
        self.table = np.full((batch, max_blocks_per_seq), -1, np.int32)

    def step(self, past, q_lens):
        """``(block_table, slot_mapping)`` for one step with these lengths."""
        slots = []
        for b, (p0, ql) in enumerate(zip(past, q_lens)):
            p0, ql = int(p0), int(ql)
            lo = max(0, p0 - self.W + 1) // self.bs          # first reachable block
            self.table[b, :lo] = -1
            for p in range(p0, p0 + ql):
                i = p // self.bs
                r = self.ring[b, i % self.N]
                live = np.nonzero(self.table[b] == r)[0]
                if any(int(j) != i for j in live):
                    raise ValueError(f"request {b}: block index {i} would overwrite live "
                                     f"block index {int(live[0])}")
                self.table[b, i] = r
                slots.append(int(r) * self.bs + p % self.bs)
        return self.table.copy(), np.asarray(slots, np.int32)


def full_cache_table(batch: int, max_blocks_per_seq: int, seed: int = 0):
    """A table that gives every (request, block index) its own physical
    block, shuffled over a pool of ``batch * max_blocks_per_seq`` blocks."""
    perm = np.random.default_rng(seed).permutation(batch * max_blocks_per_seq)
    return perm.reshape(batch, max_blocks_per_seq).astype(np.int32)


def step_tokens(seed: int, step: int, q_lens, num_heads: int, kv_num_heads: int,
                head_size: int):
    """Packed ``(cum, query, key, value)`` of one step's new tokens (fp16
    N(0, 1)), drawn from ``default_rng([seed, step])``."""
    rng = np.random.default_rng([seed, step])
    q_lens = np.asarray(q_lens, np.int64)
    cum = np.zeros(len(q_lens) + 1, np.int32)
    cum[1:] = np.cumsum(q_lens)
    T = int(cum[-1])
    q = rng.standard_normal((T, num_heads * head_size), dtype=np.float32).astype(np.float16)
    k = rng.standard_normal((T, kv_num_heads * head_size), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((T, kv_num_heads * head_size), dtype=np.float32).astype(np.float16)
    return cum, q, k, v
