"""Plain fp64 CPU oracle for paged KV append + PagedAttention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``paged_kv_cache_append_amd/csrc``) and imports nothing from it.

It writes out the plain definition of what the op computes, slowly and
visibly:

1. append: every new token's K/V row is stored at its derived slot;
2. gather: each sequence's K/V are collected from the block pool via its
   block-table row, up-cast to fp64;
3. scores: the full ``[q_len, kv_len]`` score matrix per query head;
4. softcap, then the causal / local-window mask as exclusion;
5. softmax over the admitted keys (max-subtracted) and ``P @ V``.

Sources (page title, section):

* PagedAttention -- CUDA Design Document, §4.3-§4.8 (contract, positions
  ``past_seqlens[b] + j``), §5.1 (derived write slot), §4.5 and §9 (window of W
  positions including the current one), §8.5 implementation note (softcap
  ``softcap * tanh(qk * scale / softcap)``; window ``[kv_len - W, kv_len)``),
  §12.6 (default scale ``1/sqrt(head_size)``), §18.2 (tokens past
  ``cumulative_sequence_length[batch_size]`` own nothing).
* Design: WebGPU PagedAttention, §4.1 (per-batch causal length
  ``past + q_idx + 1``, GQA grouping ``n_reps = num_heads / kv_num_heads``) and
  §7 (scatter before attention).
* GroupQueryAttention CPU Implementation Notes, "Naive Path" (QK GEMM, then
  masking/softcap/softmax, then SV GEMM, with the full score matrix).

Readings where the pages are silent (each also listed in the design notes):

* q head ``h`` reads kv head ``h // (num_heads // kv_num_heads)``.
* softcap is applied to the scaled score first; masked keys are then
  excluded (they never enter the softmax).
* RoPE (formula not printed on the pages): rotate-half pairs ``(i, i + r/2)``
  when not interleaved, ``(2i, 2i+1)`` when interleaved, angle index ``i``,
  ``x' = x*c - y*s``, ``y' = y*c + x*s``; channels ``>= r`` pass through.
  The rotated K that is stored in the fp16 pool is ``fp16(fp32(x*c - y*s))``
  (both products of fp16 numbers are exact in fp32; one fp32 rounding of the
  exact result, then one fp16 rounding).  The direction of rotation is
  parity unpinned: the pages print no formula, the tests only pin
  self-consistency properties.
* A query row with no admitted key is 0 (causal masking with W >= 1 always
  admits the query's own position; only unmapped blocks can empty a row).
* Output rows of tokens owned by no sequence are 0.
* Quantized caches (PagedAttention -- CUDA Design Document, §8.3): the
  dequantized value of a stored code is ``q * scale`` (zero point 0), with one
  scale per tensor or one per (kv head, channel).  The pages print no
  quantizer; the reading here is ``code = saturate(round_half_even(x / scale))``
  where ``x`` is the fp16 value the unquantized path would store (after
  rotary) and the division is one fp32 division: int8 saturates to
  ``[-128, 127]``, float8 e4m3fn (bias 7, no infinities, largest finite 448)
  to ``+-448``.
* Attention sink (PagedAttention -- CUDA Design Document, §6.1): the head's
  sink logit ``s_h`` joins the softmax denominator only,
  ``p_i = e^(x_i - m) / (e^(s_h - m) + sum_j e^(x_j - m))`` with
  ``m = max(s_h, max_j x_j)``; ``x`` is the score after scale and softcap
  (the sink is a logit of its own and is neither scaled nor capped).
  ``use_smooth_softmax`` without ``head_sink`` is a sink of 0 for every head
  (the page's schema lists the attribute; its §6.1 says a sink only exists
  when given, so the attribute is read as a zero-valued sink).
* QK-Norm (PagedAttention -- CUDA Design Document, §7.1-§7.2): per head,
  ``x * w / sqrt(mean(x^2) + eps)`` with one fp16 weight vector of
  ``head_size`` shared by all heads, applied to Q and to the new K before
  RoPE.  The prologue of §7.2 stages the normalized rows in an fp16 buffer
  (§7.3), so the normalized value is rounded to fp16 before it is rotated
  (and before K is quantized).  Computed here in fp64 (§7.1 asks for an fp32
  sum of squares; the kernels' fp32 result may round to a neighbouring fp16
  value, one unit in the last place).
* Latent attention (MLA, PagedAttention -- CUDA Design Document, §12.2-§12.5):
  with ``kv_cache_layout = LATENT`` there is one cache, ``kv_num_heads = 1``;
  V is the leading ``v_head_size`` channels of each K row (no value input,
  no value cache) and the output has ``v_head_size`` channels per head.
  RoPE covers channels ``[rotary_offset, rotary_offset + rotary_dim)`` of a
  head (§12.5); the pairs and angle index are those of R6 counted from the
  offset.
* Unmapped blocks (PagedAttention -- CUDA Design Document, §9.2 item 3,
  §9.3.1): a ``block_table`` entry of ``-1`` means the block is not mapped;
  every position in it is masked out of the softmax, and the derived append
  writes nothing there (as for a ``-1`` slot).  The pages name only ``-1``;
  an entry that names no block of the pool, and a position past the row's
  capacity, are read the same way here.  A row left with no admitted key is 0
  (the convention of the empty split).
* Explicit write slots (PagedAttention -- CUDA Design Document, §5.2): slot
  ``s`` is block ``s // block_size``, offset ``s % block_size``; ``-1`` writes
  nothing.  The stored K is still rotated at the token's position
  ``past[b] + j`` (the slot only says where it goes).  Tokens owned by no
  sequence write nothing, as on the derived path.  Values outside
  ``[-1, num_blocks * block_size)`` are undefined by §5.4; here they write
  nothing.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Iterable, Optional

import numpy as np


# ---------------------------------------------------------------------------
# a1 / a2: token -> (sequence, position) -> slot
# PagedAttention -- CUDA Design Document, §5.1 (derived write slot) and §18.2.
# ---------------------------------------------------------------------------

def locate_token(cum: np.ndarray, t: int):
    """Return ``(b, j)`` for packed token ``t``: the sequence ``b`` with
    ``cum[b] <= t < cum[b+1]`` and its offset ``j = t - cum[b]``; ``None`` when
    ``t >= cum[batch_size]`` (the token belongs to no sequence)."""
    B = len(cum) - 1
    for b in range(B):                       # plain scan, no search trick
        if int(cum[b]) <= t < int(cum[b + 1]):
            return b, t - int(cum[b])
    return None


def token_position(past: np.ndarray, b: int, j: int) -> int:
    """Position of the j-th new token of sequence b: ``past[b] + j``
    (PagedAttention -- CUDA Design Document, §4.8)."""
    return int(past[b]) + j


def derived_slot(block_table: np.ndarray, b: int, pos: int, block_size: int,
                 num_blocks: Optional[int] = None):
    """``(physical block, offset)`` holding position ``pos`` of sequence ``b``:
    ``block_table[b, pos // block_size]`` and ``pos % block_size``
    (PagedAttention -- CUDA Design Document, §5.1), or ``None`` when the
    position is unmapped: its table entry is ``-1`` (§9.2 item 3 and §9.3.1:
    block not mapped, every position in it masked out), names no block of a
    pool of ``num_blocks`` blocks, or lies past the row's capacity."""
    i = pos // block_size
    if i >= block_table.shape[1]:
        return None
    blk = int(block_table[b, i])
    if blk < 0 or (num_blocks is not None and blk >= num_blocks):
        return None
    return blk, pos % block_size


def mapped_keys(block_table: np.ndarray, b: int, kv_len: int, block_size: int,
                num_blocks: int) -> np.ndarray:
    """bool ``[kv_len]``: whether position ``tau`` of sequence ``b`` has a
    block (see :func:`derived_slot`).  Unmapped positions are excluded from
    the softmax like masked keys (§9.2 item 3)."""
    return np.array([derived_slot(block_table, b, tau, block_size, num_blocks) is not None
                     for tau in range(kv_len)], dtype=bool)


# ---------------------------------------------------------------------------
# a3: rotary embedding (formula not printed on the pages -- see header)
# ---------------------------------------------------------------------------

def _rotary_pairs(rotary_dim: int, interleaved: bool, offset: int = 0):
    """List of ``(first, second, angle index)`` channel pairs; the rotated
    channels start at ``offset`` (§12.5)."""
    half = rotary_dim // 2
    if interleaved:
        return [(offset + 2 * i, offset + 2 * i + 1, i) for i in range(half)]
    return [(offset + i, offset + i + half, i) for i in range(half)]


def rope_key_fp16(x16: np.ndarray, pos: int, cos16: np.ndarray, sin16: np.ndarray,
                  interleaved: bool, offset: int = 0) -> np.ndarray:
    """Rotate one fp16 head row ``x16 [D]`` at ``pos`` and round it the way it
    is stored in the fp16 pool: exact products, one fp32 rounding of their
    difference, one fp16 rounding."""
    rotary_dim = 2 * cos16.shape[1]
    out = x16.copy()
    for a, b, i in _rotary_pairs(rotary_dim, interleaved, offset):
        x = float(x16[a])
        y = float(x16[b])
        c = float(cos16[pos, i])
        s = float(sin16[pos, i])
        # products of two fp16 values are exact in fp64; the fp64 difference
        # rounded to fp32 equals the fp32-rounded exact difference (53 >= 2*24+2).
        first = np.float32(x * c - y * s)
        second = np.float32(y * c + x * s)
        out[a] = np.float16(first)
        out[b] = np.float16(second)
    return out


def rope_query_fp64(x: np.ndarray, pos: int, cos: np.ndarray, sin: np.ndarray,
                    interleaved: bool, offset: int = 0) -> np.ndarray:
    """Rotate one head row in fp64 with no rounding (used for queries, which
    are never stored)."""
    rotary_dim = 2 * cos.shape[1]
    out = np.array(x, dtype=np.float64, copy=True)
    for a, b, i in _rotary_pairs(rotary_dim, interleaved, offset):
        c = float(cos[pos, i])
        s = float(sin[pos, i])
        out[a] = float(x[a]) * c - float(x[b]) * s
        out[b] = float(x[b]) * c + float(x[a]) * s
    return out


# ---------------------------------------------------------------------------
# QK-Norm: PagedAttention -- CUDA Design Document, §7.1
# ---------------------------------------------------------------------------

QK_NORM_EPSILON = 1e-6     # §7.1 default
LAYOUT_SEPARATE, LAYOUT_LATENT = 0, 1   # kv_cache_layout (§12.3)


def rms_norm_fp16(x16: np.ndarray, w16: np.ndarray, eps: float) -> np.ndarray:
    """RMS-norm of one fp16 head row with an fp16 weight, in fp64, rounded
    to fp16: ``x[c] * w[c] / sqrt(sum_j x[j]^2 / head_size + eps)``."""
    x = x16.astype(np.float64)
    r = 1.0 / math.sqrt(float(np.sum(x * x)) / x.shape[0] + float(eps))
    return (x * r * w16.astype(np.float64)).astype(np.float16)


# ---------------------------------------------------------------------------
# quantized caches: PagedAttention -- CUDA Design Document, §8.2-§8.4
# (int8 / float8 e4m3fn codes, fp32 scales, symmetric: x = q * scale)
# ---------------------------------------------------------------------------

CACHE_FP16, CACHE_INT8, CACHE_FP8 = 0, 1, 2
QUANT_NONE, QUANT_PER_TENSOR, QUANT_PER_CHANNEL = 0, 1, 2
FP8_MAX = 448.0


def fp8_e4m3fn_value(code: int) -> float:
    """Value of one float8 e4m3fn byte: sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7f / 0xff is NaN;
    there are no infinities."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3fn_code(x: float) -> int:
    """The float8 e4m3fn byte nearest to ``x`` (ties to an even mantissa),
    saturating to +-448; exact (rational) arithmetic."""
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x))
    if a >= FP8_MAX:
        return sign | 0x7E
    best = None
    # all finite non-negative codes in increasing order of value
    for code in range(0x7F):
        v = Fraction(fp8_e4m3fn_value(code))
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and (code & 1) == 0):
            best = (d, code)
    return sign | best[1]


def fp8_e4m3fn_codes(y: np.ndarray) -> np.ndarray:
    """Vectorized :func:`fp8_e4m3fn_code` for float32 values: the nearest of
    the finite code values (ties to the even code), saturating to +-448."""
    vals = np.array([fp8_e4m3fn_value(c) for c in range(0x7F)], np.float64)   # increasing
    mids = (vals[:-1] + vals[1:]) / 2.0                                       # exact in fp64
    a = np.abs(y.astype(np.float64))
    idx = np.searchsorted(mids, a, side="left")
    tie = (idx < mids.shape[0]) & (mids[np.minimum(idx, mids.shape[0] - 1)] == a)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    idx = np.where(a >= FP8_MAX, 0x7E, idx)
    sign = np.where(np.signbit(y), 0x80, 0)
    return (sign | idx).astype(np.uint8)


def quant_scale(scale: np.ndarray, quant_type: int, kvh: int, ch: int, head_size: int) -> float:
    """The fp32 scale of channel ``ch`` of kv head ``kvh``: one value per
    tensor, or ``scale[kvh * head_size + ch]`` per channel (§8.3: shape
    ``[kv_num_heads, 1, head_size]``)."""
    flat = np.asarray(scale, np.float32).reshape(-1)       # [1] or [Hkv, (1,) D]
    if quant_type == QUANT_PER_TENSOR:
        return float(flat[0])
    return float(flat[kvh * head_size + ch])


def quantize_row(x16: np.ndarray, cache_dtype: int, scale: np.ndarray, quant_type: int,
                 kvh: int) -> np.ndarray:
    """Codes of one fp16 head row (see the header for the rounding)."""
    D = x16.shape[0]
    s = np.array([quant_scale(scale, quant_type, kvh, c, D) for c in range(D)], np.float32)
    y = x16.astype(np.float32) / s                       # one fp32 division per channel
    if cache_dtype == CACHE_INT8:
        return np.clip(np.rint(y), -128, 127).astype(np.int8)
    return fp8_e4m3fn_codes(y)


def dequantize(codes: np.ndarray, cache_dtype: int, scale: np.ndarray, quant_type: int,
               head_size: int) -> np.ndarray:
    """fp64 values ``q * scale`` of codes ``[..., Hkv, D]`` (§8.3)."""
    if cache_dtype == CACHE_INT8:
        q = codes.astype(np.float64)
    else:
        table = np.array([fp8_e4m3fn_value(c) for c in range(256)], np.float64)
        q = table[codes.astype(np.uint8)]
    Hkv = codes.shape[-2]
    if quant_type == QUANT_PER_TENSOR:
        sc = np.full((Hkv, head_size), float(np.asarray(scale, np.float32).reshape(-1)[0]),
                     np.float64)
    else:
        sc = np.asarray(scale, np.float32).astype(np.float64).reshape(Hkv, head_size)
    return q * sc


# ---------------------------------------------------------------------------
# a4: KV append (scatter new tokens into the pool, in place semantics)
# Design: WebGPU PagedAttention §7 (scatter before attention);
# PagedAttention -- CUDA Design Document §4.4 (cache outputs alias inputs).
# ---------------------------------------------------------------------------

def explicit_slot(slot_mapping: np.ndarray, t: int, block_size: int, num_blocks: int):
    """``(physical block, offset)`` of token ``t`` from an explicit slot
    mapping (PagedAttention -- CUDA Design Document, §5.2: the flat slot
    ``block * block_size + offset``), or ``None`` for ``-1`` (no write) and
    for values outside the pool."""
    s = int(slot_mapping[t])
    if s < 0 or s >= num_blocks * block_size:
        return None
    return s // block_size, s % block_size


def append_kv(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
              value: np.ndarray, cum: np.ndarray, past: np.ndarray,
              block_table: np.ndarray, *, kv_num_heads: int, head_size: int,
              cos_cache: Optional[np.ndarray] = None, sin_cache: Optional[np.ndarray] = None,
              rotary_interleaved: bool = False, slot_mapping: Optional[np.ndarray] = None,
              cache_dtype: int = CACHE_FP16, k_quant_type: int = QUANT_NONE,
              v_quant_type: int = QUANT_NONE, k_scale: Optional[np.ndarray] = None,
              v_scale: Optional[np.ndarray] = None, k_norm_weight: Optional[np.ndarray] = None,
              qk_norm_epsilon: float = QK_NORM_EPSILON, rotary_offset: int = 0,
              kv_cache_layout: int = LAYOUT_SEPARATE):
    """Return new ``(key_cache, value_cache)`` copies with every new token's
    K (RMS-normed with ``k_norm_weight`` if given, then rotated if a rotary
    table is given; §7.2 order) and V stored at its derived slot, or at
    ``slot_mapping[t]`` when a mapping is given.  With a quantized cache the
    stored rows are the codes of those fp16 rows (§8.4: quantized as they
    are scattered).  Slots that no token maps to are left byte-identical.
    With ``kv_cache_layout = LATENT`` only the key cache exists (``value``
    and ``value_cache`` are None; §12.2) and None is returned for V."""
    latent = kv_cache_layout == LAYOUT_LATENT
    kc = key_cache.copy()
    vc = None if latent else value_cache.copy()
    block_size = kc.shape[1]
    Hkv, D = kv_num_heads, head_size
    T = key.shape[0]
    for t in range(T):
        owner = locate_token(cum, t)
        if owner is None:
            continue
        b, j = owner
        pos = token_position(past, b, j)
        if slot_mapping is None:
            # an unmapped block (-1) takes no write, as a -1 slot does (§9.2 item 3)
            where = derived_slot(block_table, b, pos, block_size, kc.shape[0])
        else:
            where = explicit_slot(slot_mapping, t, block_size, kc.shape[0])
        if where is None:
            continue
        blk, off = where
        for h in range(Hkv):
            krow = key[t, h * D:(h + 1) * D]
            if k_norm_weight is not None:
                krow = rms_norm_fp16(krow, k_norm_weight, qk_norm_epsilon)
            if cos_cache is not None:
                krow = rope_key_fp16(krow, pos, cos_cache, sin_cache, rotary_interleaved,
                                     rotary_offset)
            if cache_dtype != CACHE_FP16:
                krow = quantize_row(krow, cache_dtype, k_scale, k_quant_type, h)
            kc[blk, off, h, :] = krow
            if not latent:
                vrow = value[t, h * D:(h + 1) * D]
                if cache_dtype != CACHE_FP16:
                    vrow = quantize_row(vrow, cache_dtype, v_scale, v_quant_type, h)
                vc[blk, off, h, :] = vrow
    return kc, vc


# ---------------------------------------------------------------------------
# a5 / a7: attention over the paged context
# ---------------------------------------------------------------------------

def gather_sequence(cache: np.ndarray, block_table: np.ndarray, b: int, kv_len: int) -> np.ndarray:
    """fp64 ``[kv_len, Hkv, D]``: position ``tau`` of sequence ``b`` read from
    block ``block_table[b, tau // bs]``, offset ``tau % bs``.  Unmapped
    positions (:func:`derived_slot` gives None) are not read and hold 0; the
    caller excludes them with :func:`mapped_keys`."""
    bs = cache.shape[1]
    out = np.zeros((kv_len, cache.shape[2], cache.shape[3]), np.float64)
    for tau in range(kv_len):
        where = derived_slot(block_table, b, tau, bs, cache.shape[0])
        if where is not None:
            out[tau] = cache[where]
    return out


def gather_codes(cache: np.ndarray, block_table: np.ndarray, b: int, kv_len: int) -> np.ndarray:
    """The stored codes ``[kv_len, Hkv, D]`` of sequence ``b`` (same walk as
    :func:`gather_sequence`, no conversion; unmapped positions hold code 0)."""
    bs = cache.shape[1]
    out = np.zeros((kv_len, cache.shape[2], cache.shape[3]), cache.dtype)
    for tau in range(kv_len):
        where = derived_slot(block_table, b, tau, bs, cache.shape[0])
        if where is not None:
            out[tau] = cache[where]
    return out


def effective_scale(scale: float, head_size: int) -> float:
    """``scale == 0`` selects ``1/sqrt(head_size)`` (PagedAttention -- CUDA
    Design Document, §12.6)."""
    return float(scale) if scale != 0.0 else 1.0 / math.sqrt(head_size)


def admitted(tau: np.ndarray, pos: int, local_window_size: int) -> np.ndarray:
    """Keys a query at ``pos`` may attend: ``tau <= pos`` (causal, bottom-right
    aligned) and, with a window ``W >= 1``, ``tau >= pos - W + 1`` (W positions
    including the current one)."""
    ok = tau <= pos
    if local_window_size >= 1:
        ok &= tau >= pos - local_window_size + 1
    return ok


def forward(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
            cum: np.ndarray, past: np.ndarray, block_table: np.ndarray, *,
            num_heads: int, kv_num_heads: int, head_size: int, scale: float = 0.0,
            softcap: float = 0.0, local_window_size: int = -1,
            cos_cache: Optional[np.ndarray] = None, sin_cache: Optional[np.ndarray] = None,
            rotary_interleaved: bool = False, rows: Optional[Iterable[int]] = None,
            return_probs: bool = False, cache_dtype: int = CACHE_FP16,
            k_quant_type: int = QUANT_NONE, v_quant_type: int = QUANT_NONE,
            k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
            head_sink: Optional[np.ndarray] = None, use_smooth_softmax: bool = False,
            q_norm_weight: Optional[np.ndarray] = None,
            qk_norm_epsilon: float = QK_NORM_EPSILON, rotary_offset: int = 0,
            kv_cache_layout: int = LAYOUT_SEPARATE, v_head_size: int = 0):
    """Attention output in fp64.

    ``key_cache``/``value_cache`` must already hold the new tokens (run
    :func:`append_kv` first); a quantized cache holds codes, which are
    dequantized (``q * scale``, §8.3) as they are gathered.  ``q_norm_weight``
    RMS-norms each query head before RoPE (§7); ``head_sink`` (``[H]``) or
    ``use_smooth_softmax`` adds a denominator-only logit per head (§6.1).
    With ``kv_cache_layout = LATENT`` (§12.2) V is the leading
    ``v_head_size`` channels of K (``value_cache`` is not read) and each head
    outputs ``v_head_size`` channels.
    Returns ``[T, H*DV]`` for all tokens, or ``[len(rows), H*DV]`` in the
    given order when ``rows`` is set (``DV = D`` unless latent).  With
    ``return_probs`` also returns ``{(t, h): probabilities over keys}``."""
    T = query.shape[0]
    H, Hkv, D = num_heads, kv_num_heads, head_size
    g = H // Hkv
    sigma = effective_scale(scale, D)
    latent = kv_cache_layout == LAYOUT_LATENT
    DV = v_head_size if latent and v_head_size else D
    row_list = list(range(T)) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(row_list), H * DV), np.float64)
    probs = {}

    # group the requested rows by owning sequence so each context is gathered once
    by_seq = {}
    for n, t in enumerate(row_list):
        owner = locate_token(cum, t)
        if owner is None:
            continue                          # owned by no sequence: row stays 0
        b, j = owner
        by_seq.setdefault(b, []).append((n, t, j))

    sink = None
    if head_sink is not None:
        sink = np.asarray(head_sink).astype(np.float64).reshape(H)
    elif use_smooth_softmax:
        sink = np.zeros(H, np.float64)

    for b, items in by_seq.items():
        q_len = int(cum[b + 1]) - int(cum[b])
        kv_len = int(past[b]) + q_len
        if cache_dtype != CACHE_FP16:
            K = dequantize(gather_codes(key_cache, block_table, b, kv_len), cache_dtype, k_scale,
                           k_quant_type, D)
            if not latent:
                V = dequantize(gather_codes(value_cache, block_table, b, kv_len), cache_dtype,
                               v_scale, v_quant_type, D)
        else:
            K = gather_sequence(key_cache, block_table, b, kv_len)
            if not latent:
                V = gather_sequence(value_cache, block_table, b, kv_len)
        if latent:
            V = K[:, :, :DV]                                   # V is a view of K (§12.2)
        tau = np.arange(kv_len)
        n_idx = [n for n, _, _ in items]
        positions = [token_position(past, b, j) for _, _, j in items]
        # queries [n_rows, H, D] in fp64, rotated at their position if asked
        Q = np.empty((len(items), H, D), np.float64)
        for r, (_, t, _) in enumerate(items):
            if q_norm_weight is not None:
                qrow = np.stack([rms_norm_fp16(query[t, h * D:(h + 1) * D], q_norm_weight,
                                               qk_norm_epsilon) for h in range(H)])
                qrow = qrow.astype(np.float64)
            else:
                qrow = query[t].astype(np.float64).reshape(H, D)
            if cos_cache is not None:
                for h in range(H):
                    qrow[h] = rope_query_fp64(qrow[h], positions[r], cos_cache, sin_cache,
                                              rotary_interleaved, rotary_offset)
            Q[r] = qrow
        # keys in unmapped blocks are masked out like keys outside the window
        mapped = mapped_keys(block_table, b, kv_len, key_cache.shape[1], key_cache.shape[0])
        mask = np.stack([admitted(tau, p, local_window_size) & mapped for p in positions])
        for h in range(H):
            kvh = h // g
            S = sigma * (Q[:, h, :] @ K[:, kvh, :].T)          # full score matrix
            if softcap > 0.0:
                S = softcap * np.tanh(S / softcap)
            S = np.where(mask, S, -np.inf)                     # exclusion
            O = np.zeros((len(items), DV), np.float64)
            for r in range(len(items)):
                if not mask[r].any():
                    continue                                   # fully masked -> 0
                m = S[r].max()
                if sink is not None:
                    m = max(m, sink[h])
                e = np.exp(S[r] - m)
                den = e.sum() + (math.exp(sink[h] - m) if sink is not None else 0.0)
                p = e / den
                if sink is None:
                    assert abs(p.sum() - 1.0) < 1e-12
                O[r] = p @ V[:, kvh, :]
                if return_probs:
                    probs[(items[r][1], h)] = p
            out[n_idx, h * DV:(h + 1) * DV] = O
    if return_probs:
        return out, probs
    return out
