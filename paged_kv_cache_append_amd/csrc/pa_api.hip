// Host side of the C ABI: validation, launch planning and kernel launches.
//
// Validation follows the consolidated rules of PagedAttention -- CUDA Design
// Document, section 15 (every violation names the offending argument and the
// expected value); planning follows section 4.7: only static shapes,
// attributes and the optional replay-wide bounds choose kernels and size
// grids/workspace -- device-resident lengths never reach the host, so a
// captured stream stays valid while lengths change.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pa.h"
#include "../../include/pa_testing.h"
#include "pa_internal.h"

namespace {

thread_local std::string g_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// ---- per-kernel timing (benchmarks) ---------------------------------------
struct Timing {
  std::mutex mu;
  bool enabled = false;
  std::vector<hipEvent_t> events;   // pairs
  std::vector<int> stage;           // per pair
  size_t used = 0;                  // pairs recorded
};
Timing g_timing;
}  // namespace

namespace pa {
thread_local LaunchEvents g_launch_events;
}  // namespace pa

namespace {

struct StageScope {
  int slot = -1;
  StageScope(int stg, hipStream_t) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.enabled || g_timing.used >= g_timing.stage.size()) return;
    slot = (int)g_timing.used++;
    g_timing.stage[slot] = stg;
    pa::g_launch_events = {g_timing.events[2 * slot], g_timing.events[2 * slot + 1]};
  }
  ~StageScope() { pa::g_launch_events = {}; }
};

// ---- validation --------------------------------------------------------------
const char* quant_name(int q) {
  return q == PA_QUANT_NONE ? "NONE" : q == PA_QUANT_PER_TENSOR ? "PER_TENSOR" : "PER_CHANNEL";
}

// One cache's quant type against its scale (PagedAttention -- CUDA Design
// Document, section 8.7: a quant type other than NONE needs its scale, NONE
// forbids one; a per-channel scale is read 16 bytes at a time).
pa_status check_scale(const char* which, int quant, const float* scale) {
  if (quant < PA_QUANT_NONE || quant > PA_QUANT_PER_CHANNEL)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "%s_quant_type: expected 0 (NONE), 1 (PER_TENSOR) or 2 (PER_CHANNEL), got %d",
                which, quant);
  if (quant == PA_QUANT_NONE && scale)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s_scale: given but %s_quant_type is NONE", which,
                which);
  if (quant != PA_QUANT_NONE && !scale)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s_scale: required when %s_quant_type is %s", which,
                which, quant_name(quant));
  const uintptr_t align = quant == PA_QUANT_PER_CHANNEL ? 16 : 4;
  if ((reinterpret_cast<uintptr_t>(scale) & (align - 1)) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s_scale: expected %d-byte alignment for %s", which,
                (int)align, quant_name(quant));
  return PA_OK;
}

// Cache element type against the quant types (section 8.7: a quantized cache
// needs both quant types other than NONE; an fp16 cache needs both NONE).
pa_status check_quant(const pa_attn_params* p, const pa_paged_kv* kv) {
  if (p->cache_dtype < PA_CACHE_FP16 || p->cache_dtype > PA_CACHE_FP8_E4M3FN)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "cache_dtype: expected 0 (fp16), 1 (int8) or 2 (float8 e4m3fn), got %d",
                p->cache_dtype);
  pa_status st = check_scale("k", p->k_quant_type, kv->k_scale);
  if (st == PA_OK) st = check_scale("v", p->v_quant_type, kv->v_scale);
  if (st != PA_OK) return st;
  const bool quantized = p->cache_dtype != PA_CACHE_FP16;
  if (p->kv_cache_layout == PA_LAYOUT_LATENT) {
    // one physical cache, described by k_scale alone (section 8.3, 12.10)
    if (p->v_quant_type != PA_QUANT_NONE || kv->v_scale)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "v_quant_type/v_scale: expected NONE/NULL with kv_cache_layout LATENT");
    if (quantized != (p->k_quant_type != PA_QUANT_NONE))
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "k_quant_type: expected %s with this cache_dtype, got %s",
                  quantized ? "PER_TENSOR or PER_CHANNEL" : "NONE", quant_name(p->k_quant_type));
    return PA_OK;
  }
  if (!quantized && (p->k_quant_type != PA_QUANT_NONE || p->v_quant_type != PA_QUANT_NONE))
    return fail(PA_ERR_INVALID_ARGUMENT,
                "k_quant_type/v_quant_type: expected NONE with an fp16 cache, got %s/%s",
                quant_name(p->k_quant_type), quant_name(p->v_quant_type));
  if (quantized && (p->k_quant_type == PA_QUANT_NONE || p->v_quant_type == PA_QUANT_NONE))
    return fail(PA_ERR_INVALID_ARGUMENT,
                "k_quant_type/v_quant_type: expected PER_TENSOR or PER_CHANNEL with a quantized "
                "cache_dtype, got %s/%s",
                quant_name(p->k_quant_type), quant_name(p->v_quant_type));
  return PA_OK;
}

// Attention sink and QK-Norm (PagedAttention -- CUDA Design Document,
// section 6.4 and section 7.4: both norm weights or neither, epsilon > 0).
pa_status check_sink_norm(const pa_attn_params* p) {
  if (p->use_smooth_softmax != 0 && p->use_smooth_softmax != 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "use_smooth_softmax: expected 0 or 1, got %d",
                p->use_smooth_softmax);
  if ((reinterpret_cast<uintptr_t>(p->head_sink) & 1) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "head_sink: expected 2-byte alignment");
  if ((p->q_norm_weight == nullptr) != (p->k_norm_weight == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "q_norm_weight/k_norm_weight: expected both or neither");
  if (!aligned16(p->q_norm_weight) || !aligned16(p->k_norm_weight))
    return fail(PA_ERR_INVALID_ARGUMENT, "q_norm_weight/k_norm_weight: expected 16-byte alignment");
  if (!std::isfinite(p->qk_norm_epsilon) || p->qk_norm_epsilon < 0.f)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "qk_norm_epsilon: expected 0 (default 1e-6) or a finite value > 0, got %g",
                (double)p->qk_norm_epsilon);
  return PA_OK;
}

// QK-Norm sums a head row's squares across D/8 lanes of a wave.
pa_status check_norm_support(const pa_attn_params* p) {
  if (p->k_norm_weight && p->head_size != 64 && p->head_size != 128 && p->head_size != 256)
    return fail(PA_ERR_UNSUPPORTED, "QK-Norm with head_size %d: served for 64, 128 and 256",
                p->head_size);
  return PA_OK;
}

float norm_epsilon(const pa_attn_params* p) {
  return p->qk_norm_epsilon > 0.f ? p->qk_norm_epsilon : 1e-6f;
}

// Latent layout (MLA) and offset RoPE (PagedAttention -- CUDA Design
// Document, section 12.10).
int effective_v_head_size(const pa_attn_params* p) {
  return p->kv_cache_layout == PA_LAYOUT_LATENT && p->v_head_size != 0 ? p->v_head_size
                                                                       : p->head_size;
}

pa_status check_layout(const pa_attn_params* p, const pa_paged_kv* kv) {
  if (p->kv_cache_layout != PA_LAYOUT_SEPARATE && p->kv_cache_layout != PA_LAYOUT_LATENT)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "kv_cache_layout: expected 0 (SEPARATE) or 1 (LATENT), got %d",
                p->kv_cache_layout);
  if (p->v_head_size < 0 || p->v_head_size > p->head_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "v_head_size: expected 0..head_size (%d), got %d",
                p->head_size, p->v_head_size);
  if (p->rotary_offset < 0 || p->rotary_offset % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "rotary_offset: expected a non-negative multiple of 8, got %d", p->rotary_offset);
  if (p->kv_cache_layout == PA_LAYOUT_SEPARATE) {
    if (p->v_head_size != 0 && p->v_head_size != p->head_size)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "v_head_size: %d != head_size requires kv_cache_layout LATENT", p->v_head_size);
    if (!kv->value_cache)
      return fail(PA_ERR_INVALID_ARGUMENT, "value_cache: expected non-NULL");
    return PA_OK;
  }
  if (p->kv_num_heads != 1)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "kv_num_heads: expected 1 with kv_cache_layout LATENT, got %d", p->kv_num_heads);
  if (kv->value_cache)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "value_cache: expected NULL with kv_cache_layout LATENT (V is a view of K)");
  if (effective_v_head_size(p) != p->head_size && p->scale == 0.f)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "scale: an explicit scale is required when v_head_size != head_size");
  if (p->head_sink || p->use_smooth_softmax || p->q_norm_weight || p->k_norm_weight)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "head_sink/use_smooth_softmax/QK-Norm: not allowed with kv_cache_layout LATENT");
  if (p->do_rotary && p->rotary_offset < effective_v_head_size(p))
    return fail(PA_ERR_INVALID_ARGUMENT,
                "rotary_offset: expected >= v_head_size (%d) with kv_cache_layout LATENT, so "
                "that RoPE leaves the V channels alone, got %d",
                effective_v_head_size(p), p->rotary_offset);
  return PA_OK;
}

pa_status check_common(const pa_attn_params* p, const pa_paged_kv* kv) {
  if (!p) return fail(PA_ERR_INVALID_ARGUMENT, "params: expected non-NULL");
  if (!kv) return fail(PA_ERR_INVALID_ARGUMENT, "kv: expected non-NULL");
  if (p->num_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads: expected > 0, got %d", p->num_heads);
  if (p->kv_num_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_num_heads: expected > 0, got %d", p->kv_num_heads);
  if (p->num_heads % p->kv_num_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "num_heads: expected a multiple of kv_num_heads (%d), got %d", p->kv_num_heads,
                p->num_heads);
  if (p->head_size <= 0 || p->head_size % 8 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "head_size: expected a positive multiple of 8, got %d",
                p->head_size);
  if (p->block_size < 16 || (p->block_size & (p->block_size - 1)) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "block_size: expected a power of two >= 16, got %d",
                p->block_size);
  if (!std::isfinite(p->scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "scale: expected a finite value");
  if (!std::isfinite(p->softcap) || p->softcap < 0.f)
    return fail(PA_ERR_INVALID_ARGUMENT, "softcap: expected a finite value >= 0, got %g",
                (double)p->softcap);
  if (p->local_window_size != -1 && p->local_window_size < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "local_window_size: expected -1 or >= 1, got %d",
                p->local_window_size);
  if (p->do_rotary != 0 && p->do_rotary != 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "do_rotary: expected 0 or 1, got %d", p->do_rotary);
  if (p->rotary_interleaved != 0 && p->rotary_interleaved != 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "rotary_interleaved: expected 0 or 1, got %d",
                p->rotary_interleaved);
  if (p->num_heads > 65535)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_heads: expected <= 65535, got %d", p->num_heads);
  if (kv->batch_size <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "batch_size: expected > 0, got %d", kv->batch_size);
  if (kv->token_count < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "token_count: expected >= 0, got %d", kv->token_count);
  if (kv->num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "num_blocks: expected > 0, got %lld",
                (long long)kv->num_blocks);
  if (kv->num_blocks > (((int64_t)1 << 32) - 1) / p->block_size)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "num_blocks: expected num_blocks * block_size < 2^32 slots, got %lld blocks",
                (long long)kv->num_blocks);
  if (kv->max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq: expected > 0, got %d",
                kv->max_blocks_per_seq);
  if ((int64_t)kv->max_blocks_per_seq * p->block_size > (int64_t)1 << 30)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "max_blocks_per_seq * block_size: expected <= 2^30 positions");
  if (!kv->key_cache) return fail(PA_ERR_INVALID_ARGUMENT, "key_cache: expected non-NULL");
  if (!aligned16(kv->key_cache) || !aligned16(kv->value_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "key_cache/value_cache: expected 16-byte alignment");
  if (!kv->block_table) return fail(PA_ERR_INVALID_ARGUMENT, "block_table: expected non-NULL");
  if (!kv->cumulative_sequence_length)
    return fail(PA_ERR_INVALID_ARGUMENT, "cumulative_sequence_length: expected non-NULL");
  if (!kv->past_seqlens) return fail(PA_ERR_INVALID_ARGUMENT, "past_seqlens: expected non-NULL");
  pa_status st = check_sink_norm(p);
  if (st != PA_OK) return st;
  if ((st = check_layout(p, kv)) != PA_OK) return st;
  return check_quant(p, kv);
}

pa_status check_rotary(const pa_attn_params* p, const pa_paged_kv* kv, const void* cos_cache,
                       const void* sin_cache, int32_t rows, int32_t dim) {
  if ((cos_cache == nullptr) != (sin_cache == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache/sin_cache: expected both or neither");
  if (p->do_rotary) {
    if (!cos_cache)
      return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache/sin_cache: required when do_rotary = 1");
    if (dim <= 0 || dim % 2 != 0 || dim + p->rotary_offset > p->head_size)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "rotary_dim: expected an even value in [2, head_size - rotary_offset = %d], "
                  "got %d",
                  p->head_size - p->rotary_offset, dim);
    const int64_t need = (int64_t)kv->max_blocks_per_seq * p->block_size;
    if (rows < need)
      return fail(PA_ERR_INVALID_ARGUMENT,
                  "rotary_rows: expected >= max_blocks_per_seq * block_size = %lld, got %d",
                  (long long)need, rows);
    if (!aligned16(cos_cache) || !aligned16(sin_cache))
      return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache/sin_cache: expected 16-byte alignment");
  } else if (cos_cache) {
    return fail(PA_ERR_INVALID_ARGUMENT, "cos_cache/sin_cache: given but do_rotary = 0");
  }
  return PA_OK;
}

// Forced routing of the testing entry points (pa_testing.h); all zeros is the
// automatic choice of pa_forward.
pa_routing auto_routing() {
  pa_routing r;
  r.path = r.split_tokens = r.prefill_pieces = r.prefill_kernel = 0;
  return r;
}

pa_status check_routing(const pa_routing* r) {
  if (r->path < 0 || r->path > 2)
    return fail(PA_ERR_INVALID_ARGUMENT, "path: expected 0, 1 or 2, got %d", r->path);
  if (r->prefill_pieces < 0 || r->prefill_pieces > pa::kPrefillChunks)
    return fail(PA_ERR_INVALID_ARGUMENT, "prefill_pieces: expected 0..%d, got %d",
                pa::kPrefillChunks, r->prefill_pieces);
  if (r->prefill_kernel < 0 || r->prefill_kernel > 3)
    return fail(PA_ERR_INVALID_ARGUMENT, "prefill_kernel: expected 0..3, got %d",
                r->prefill_kernel);
  if (r->split_tokens < 0 || r->split_tokens % 64 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "split_tokens: expected 0 or a multiple of 64, got %d",
                r->split_tokens);
  return PA_OK;
}

// Each cache is small enough for 32-bit byte offsets (buffer addressing).
bool pool_fits_32bit(const pa_attn_params* p, const pa_paged_kv* kv) {
  return kv->num_blocks * p->block_size * p->kv_num_heads * p->head_size * 2 <
         ((int64_t)1 << 32) - 16;
}
// The 8-wave prefill kernel serves head_size 256 and addresses the caches
// with 32-bit byte offsets.
bool rows16_prefill_fits(const pa_attn_params* p, const pa_paged_kv* kv) {
  return p->head_size == 256 && pool_fits_32bit(p, kv);
}
// The 8-wave kernel of 32 rows per wave: the same shapes.
bool rows32_prefill_fits(const pa_attn_params* p, const pa_paged_kv* kv) {
  return rows16_prefill_fits(p, kv);
}
// Prefill kernel of a forward: 1 = 4-wave, 2 = 8-wave of 16 rows per wave
// (only by the testing hook), 3 = 8-wave of 32 rows per wave.
int prefill_kernel_of(const pa_attn_params* p, const pa_paged_kv* kv, const pa_routing& rt) {
  if (rt.prefill_kernel > 0) return rt.prefill_kernel;
  return rows32_prefill_fits(p, kv) ? 3 : 1;
}

pa_status check_kernel_support(const pa_attn_params* p, const pa_paged_kv* kv,
                               const pa_routing& rt) {
  if (p->kv_cache_layout == PA_LAYOUT_LATENT) {
    if (p->head_size != pa::kMlaHeadSize || effective_v_head_size(p) != pa::kMlaVHeadSize)
      return fail(PA_ERR_UNSUPPORTED,
                  "kv_cache_layout LATENT: served for head_size %d with v_head_size %d, got "
                  "%d/%d",
                  pa::kMlaHeadSize, pa::kMlaVHeadSize, p->head_size, effective_v_head_size(p));
    if (p->cache_dtype != PA_CACHE_FP16)
      return fail(PA_ERR_UNSUPPORTED, "kv_cache_layout LATENT: served for fp16 caches");
    if (rt.path == 2)
      return fail(PA_ERR_UNSUPPORTED,
                  "path 2: the latent kernel serves every token (path 0 or 1)");
    if (kv->num_blocks * p->block_size * p->head_size * 2 > (int64_t)pa::kMlaZeroRow)
      return fail(PA_ERR_UNSUPPORTED,
                  "kv_cache_layout LATENT: expected a cache of at most 4 GiB - 4 KiB");
    return PA_OK;
  }
  if (p->head_size != 64 && p->head_size != 128 && p->head_size != 256)
    return fail(PA_ERR_UNSUPPORTED,
                "head_size %d: the kernels serve head_size 64, 128 and 256", p->head_size);
  if (rt.prefill_kernel == 2 && !rows16_prefill_fits(p, kv))
    return fail(PA_ERR_UNSUPPORTED,
                "prefill_kernel 2: expected head_size 256 and caches smaller than 4 GiB");
  if (rt.prefill_kernel == 3 && !rows32_prefill_fits(p, kv))
    return fail(PA_ERR_UNSUPPORTED,
                "prefill_kernel 3: expected head_size 256 and caches smaller than 4 GiB");
  return PA_OK;
}

// ---- planning ----------------------------------------------------------------
constexpr int64_t kTargetItems = 32768;   // decode work items aimed at (split length choice)
// The latent kernel runs 4 waves per CU and each item's partials are 16 heads
// x 512 channels: fewer, longer splits (about 4 items per wave slot).
constexpr int64_t kTargetItemsLatent = 4096;

struct Plan {
  bool token_mode = true;    // decode rows are tokens (else requests with q_len == 1)
  bool prefill = false;
  bool listed = false;       // decode items come from the device-built list
  int rows = 0;
  int g = 1, chunk_heads = 1, head_chunks = 1;
  int split_tokens = 256;
  int max_splits = 1;
  int prefill_tiles = 0;     // tile slots (grid.x = tiles * prefill_chunks + 1)
  int prefill_chunks = 1;    // key-range pieces per prefill tile
  int prefill_kernel = 1;    // prefill_kernel_of
  int prefill_rows = pa::kPrefillRows;   // rows of a tile slot
  size_t off_ml = 0, off_entries = 0, off_count = 0, off_rows = 0;
  size_t off_pf_o = 0, off_pf_ml = 0;
  size_t off_qn = 0;         // QK-Norm: normalized queries, fp16 [T, H*D]
  bool q_norm = false;
  size_t ws_bytes = 0;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

Plan make_plan(const pa_attn_params* p, const pa_paged_kv* kv, const pa_routing& rt, int32_t mq,
               int32_t mk) {
  Plan pl;
  const int T = kv->token_count, B = kv->batch_size;
  pl.g = p->num_heads / p->kv_num_heads;
  for (int c = std::min(pl.g, pa::kDecodeMaxHeads); c >= 1; --c)
    if (pl.g % c == 0) {
      pl.chunk_heads = c;
      break;
    }
  pl.head_chunks = pl.g / pl.chunk_heads;
  if (rt.path == 1 || p->kv_cache_layout == PA_LAYOUT_LATENT)
    pl.token_mode = true;   // latent caches: one kernel serves every token
  else if (rt.path == 2)
    pl.token_mode = false;
  else
    pl.token_mode = T <= B;   // static shape test: a heuristic, never a correctness input
  pl.prefill = !pl.token_mode;
  pl.rows = pl.token_mode ? T : B;

  const int64_t cap = (int64_t)kv->max_blocks_per_seq * p->block_size;
  int64_t span = cap;                                   // static key-range extent
  if (p->local_window_size > 0 && p->local_window_size < span) span = p->local_window_size;
  if (rt.split_tokens > 0) {
    pl.split_tokens = rt.split_tokens;
  } else {
    // split length from static shapes only, so results do not depend on the bounds
    const int64_t items = std::max<int64_t>(1, (int64_t)pl.rows * p->kv_num_heads * pl.head_chunks);
    const int64_t target =
        p->kv_cache_layout == PA_LAYOUT_LATENT ? kTargetItemsLatent : kTargetItems;
    int64_t st = (items * span + target - 1) / target;
    st = std::max<int64_t>(st, (span + pa::kDecodeMaxSplits - 1) / pa::kDecodeMaxSplits);
    // beside a prefill, which holds part of the CUs for most of the decode,
    // fewer and longer items cost less than finer balance gains (partials,
    // merge work, per-item start-up)
    st = std::max<int64_t>(st, pl.prefill ? 256 : 128);
    st = (st + 63) / 64 * 64;
    pl.split_tokens = (int)std::min<int64_t>(st, 1 << 30);
  }
  int64_t kv_ext = mk > 0 ? std::min<int64_t>(mk, cap) : cap;   // bound only trims the grid
  if (p->local_window_size > 0) kv_ext = std::min<int64_t>(kv_ext, p->local_window_size);
  pl.max_splits = (int)std::max<int64_t>(1, (kv_ext + pl.split_tokens - 1) / pl.split_tokens);
  pl.listed = pl.max_splits > 1;
  size_t cur = 0;
  if (pl.listed) {
    const size_t per = (size_t)pl.rows * p->num_heads * pl.max_splits;
    pl.off_ml = align256(per * effective_v_head_size(p) * sizeof(float));
    pl.off_entries = pl.off_ml + align256(per * 2 * sizeof(float));
    pl.off_count = pl.off_entries + align256((size_t)pl.rows * pl.max_splits * sizeof(pa::DecodeEntry));
    pl.off_rows = pl.off_count + 256;
    cur = pl.off_rows + align256((size_t)pl.rows * sizeof(pa::RowSplit));
  }
  if (pl.prefill) {
    const int64_t mql = mq > 0 ? std::min<int64_t>(mq, T) : T;
    pl.prefill_kernel = prefill_kernel_of(p, kv, rt);
    pl.prefill_rows = pl.prefill_kernel == 3 ? 2 * pa::kPrefillRows : pa::kPrefillRows;
    const int64_t tr = pl.prefill_rows;
    const int64_t per_req = (mql * pl.g + tr - 1) / tr;
    const int64_t by_tokens = ((int64_t)T * pl.g + tr - 1) / tr + B;
    pl.prefill_tiles = (int)std::min<int64_t>(std::min<int64_t>((int64_t)B * per_req, by_tokens),
                                              (int64_t)1 << 28);
    // Few (tile, kv head) items leave most of the chip idle while each tile
    // walks its whole key range: then long tiles' key ranges are cut into
    // pieces of about kPrefillPieceTiles key tiles (at most kPrefillChunks),
    // computed by separate workgroups and combined by a merge kernel.  Static
    // shapes decide whether pieces are allowed; the device cuts by length.
    const int64_t est_items = ((int64_t)T * pl.g + tr - 1) / tr * p->kv_num_heads;
    const bool long_keys = cap >= 4 * pa::kPrefillPieceTiles * 64;
    pl.prefill_chunks = rt.prefill_pieces > 0 ? rt.prefill_pieces
                        : est_items < pa::kPrefillSplitItems && long_keys ? pa::kPrefillChunks
                                                                          : 1;
    if (pl.prefill_chunks > 1) {
      const size_t rows = (size_t)T * p->num_heads * pl.prefill_chunks;
      pl.off_pf_o = cur;
      pl.off_pf_ml = pl.off_pf_o + align256(rows * p->head_size * sizeof(float));
      cur = pl.off_pf_ml + align256(rows * 2 * sizeof(float));
    }
  }
  if (p->q_norm_weight) {
    pl.q_norm = true;
    pl.off_qn = cur;
    cur += align256((size_t)T * p->num_heads * p->head_size * sizeof(uint16_t));
  }
  pl.ws_bytes = cur;
  return pl;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// A second stream per (thread, device): a batch with both prefill and decode
// rows runs the prefill launches on it, forked from and joined back into the
// caller's stream by events, so the MFMA-bound prefill tiles share the chip
// with the HBM-bound decode workers instead of running after them.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

pa_status side_stream(hipStream_t main, SideStream** out) {
  thread_local SideStream per_dev[64];
  int dev = 0;
  hipError_t e = main ? hipStreamGetDevice(main, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "stream device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PA_ERR_DEVICE, "device index %d out of range", dev);
  SideStream& x = per_dev[dev];
  if (!x.st) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess || (e = hipSetDevice(dev)) != hipSuccess)
      return fail(PA_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(e));
    SideStream n;
    e = hipStreamCreateWithFlags(&n.st, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      if (n.st) (void)hipStreamDestroy(n.st);
      if (n.fork) (void)hipEventDestroy(n.fork);
      return fail(PA_ERR_DEVICE, "side stream creation: %s", hipGetErrorString(e));
    }
    x = n;
  }
  *out = &x;
  return PA_OK;
}

pa_status check_plan(const Plan& pl) {
  if (pl.max_splits > pa::kDecodeMaxSplits)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "split_tokens: %d gives %d splits; expected at most %d", pl.split_tokens,
                pl.max_splits, pa::kDecodeMaxSplits);
  return PA_OK;
}

pa::SeqLayout layout(const pa_attn_params* p, const pa_paged_kv* kv) {
  pa::SeqLayout s;
  s.cum = kv->cumulative_sequence_length;
  s.past = kv->past_seqlens;
  s.block_table = kv->block_table;
  s.batch = kv->batch_size;
  s.tokens = kv->token_count;
  s.maxblk = kv->max_blocks_per_seq;
  s.block_shift = log2_exact(p->block_size);
  s.num_blocks = kv->num_blocks;
  return s;
}

pa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ---- the workspace of pa_forward_noalloc -------------------------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// (PA_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code its name is
// only a stand-in; the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is passed
// to kernels.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

struct ScratchAddresses {
  std::mutex mu;
  void* ptr[64] = {};
};
ScratchAddresses g_scratch;

pa_status scratch_address(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_DEVICE, "stream device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PA_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess || (e = hipSetDevice(dev)) != hipSuccess)
      return fail(PA_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = hipSetDevice(cur);
    if (e != hipSuccess)
      return fail(PA_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (back != hipSuccess) return fail(PA_ERR_DEVICE, "hipSetDevice: %s", hipGetErrorString(back));
    if (!p) return fail(PA_ERR_DEVICE, "hipGetSymbolAddress(scratch): null address");
    g_scratch.ptr[dev] = p;
  }
  *out = g_scratch.ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

pa_status pa_append_kv(const pa_attn_params* params, const pa_paged_kv* kv, const void* key,
                       const void* value, const void* cos_cache, const void* sin_cache,
                       int32_t rotary_rows, int32_t rotary_dim, void* stream) {
  g_error.clear();
  pa_status st = check_common(params, kv);
  if (st != PA_OK) return st;
  if ((st = check_rotary(params, kv, cos_cache, sin_cache, rotary_rows, rotary_dim)) != PA_OK)
    return st;
  if (kv->token_count == 0) return PA_OK;
  if ((st = check_norm_support(params)) != PA_OK) return st;
  const bool latent = params->kv_cache_layout == PA_LAYOUT_LATENT;
  if (!key || (!value && !latent))
    return fail(PA_ERR_INVALID_ARGUMENT, "key/value: expected non-NULL");
  if (latent && value)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "value: expected NULL with kv_cache_layout LATENT (V is a view of K)");
  if (!aligned16(key) || !aligned16(value))
    return fail(PA_ERR_INVALID_ARGUMENT, "key/value: expected 16-byte alignment");
  if ((reinterpret_cast<uintptr_t>(kv->slot_mapping) & 3) != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping: expected 4-byte alignment");
  pa::AppendArgs a;
  a.s = layout(params, kv);
  a.slot_mapping = kv->slot_mapping;
  a.key = static_cast<const uint16_t*>(key);
  a.value = static_cast<const uint16_t*>(value);
  a.key_cache = static_cast<uint16_t*>(kv->key_cache);
  a.value_cache = static_cast<uint16_t*>(kv->value_cache);
  a.cos = static_cast<const uint16_t*>(cos_cache);
  a.sin = static_cast<const uint16_t*>(sin_cache);
  a.kv_heads = params->kv_num_heads;
  a.head_size = params->head_size;
  a.rotary_dim = params->do_rotary ? rotary_dim : 0;
  a.rotary_interleaved = params->rotary_interleaved;
  a.rotary_rows = params->do_rotary ? rotary_rows : 0;
  a.cache_dtype = params->cache_dtype;
  a.k_quant = params->k_quant_type;
  a.v_quant = params->v_quant_type;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.k_norm = static_cast<const uint16_t*>(params->k_norm_weight);
  a.norm_eps = norm_epsilon(params);
  a.rotary_offset = params->do_rotary ? params->rotary_offset : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope scope(PA_STAGE_APPEND, s);
  return device_status(pa::launch_append(a, s), "append kernel launch");
}

static pa_status workspace_bytes_impl(const pa_attn_params* params, const pa_paged_kv* kv,
                                      const pa_routing* routing, int32_t mq, int32_t mk,
                                      size_t* bytes) {
  g_error.clear();
  if (!bytes) return fail(PA_ERR_INVALID_ARGUMENT, "bytes: expected non-NULL");
  *bytes = 0;
  pa_status st = check_common(params, kv);
  if (st != PA_OK) return st;
  if (!routing) return fail(PA_ERR_INVALID_ARGUMENT, "routing: expected non-NULL");
  if ((st = check_routing(routing)) != PA_OK) return st;
  if (mq < 0 || mk < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_query_len_bound/max_kv_len_bound: expected >= 0");
  if (kv->token_count == 0) return PA_OK;
  const Plan pl = make_plan(params, kv, *routing, mq, mk);
  if ((st = check_plan(pl)) != PA_OK) return st;
  *bytes = pl.ws_bytes;
  return PA_OK;
}

pa_status pa_forward_workspace_bytes(const pa_attn_params* params, const pa_paged_kv* kv,
                                     int32_t mq, int32_t mk, size_t* bytes) {
  const pa_routing rt = auto_routing();
  return workspace_bytes_impl(params, kv, &rt, mq, mk, bytes);
}

pa_status pa_forward_workspace_bytes_routed(const pa_attn_params* params, const pa_paged_kv* kv,
                                            const pa_routing* routing, int32_t mq, int32_t mk,
                                            size_t* bytes) {
  return workspace_bytes_impl(params, kv, routing, mq, mk, bytes);
}

pa_status pa_describe_plan(const pa_attn_params* params, const pa_paged_kv* kv,
                           const pa_routing* routing, int32_t mq, int32_t mk, char* buf,
                           size_t len) {
  g_error.clear();
  pa_status st = check_common(params, kv);
  if (st != PA_OK) return st;
  const pa_routing rt = routing ? *routing : auto_routing();
  if ((st = check_routing(&rt)) != PA_OK) return st;
  if (!buf || len == 0) return fail(PA_ERR_INVALID_ARGUMENT, "buf: expected non-NULL, len > 0");
  const Plan pl = make_plan(params, kv, rt, mq, mk);
  snprintf(buf, len,
           "mode=%s cache=%s rows=%d head_chunks=%d g=%d chunk_heads=%d split_tokens=%d "
           "max_splits=%d listed=%d prefill_grid=(%d,%d) prefill_chunks=%d q_norm=%d "
           "workspace=%zu",
           pl.token_mode ? "token" : "request",
           params->cache_dtype == PA_CACHE_INT8  ? "int8"
           : params->cache_dtype == PA_CACHE_FP8_E4M3FN ? "fp8e4m3fn"
                                                       : "fp16", pl.rows, params->kv_num_heads * pl.head_chunks,
           pl.g, pl.chunk_heads, pl.split_tokens, pl.max_splits, pl.listed ? 1 : 0,
           pl.prefill ? pl.prefill_tiles * pl.prefill_chunks + 1 : 0,
           pl.prefill ? params->kv_num_heads : 0, pl.prefill ? pl.prefill_chunks : 0,
           pl.q_norm ? 1 : 0, pl.ws_bytes);
  return PA_OK;
}

static pa_status forward_impl(const pa_attn_params* params, const pa_paged_kv* kv,
                               const pa_routing* routing, const void* query,
                               const void* cos_cache, const void* sin_cache, int32_t rotary_rows,
                               int32_t rotary_dim, int32_t mq, int32_t mk, void* workspace,
                               size_t workspace_bytes, void* out, void* stream,
                               bool one_stream = false) {
  g_error.clear();
  pa_status st = check_common(params, kv);
  if (st != PA_OK) return st;
  if (!routing) return fail(PA_ERR_INVALID_ARGUMENT, "routing: expected non-NULL");
  if ((st = check_routing(routing)) != PA_OK) return st;
  const pa_routing& rt = *routing;
  if ((st = check_rotary(params, kv, cos_cache, sin_cache, rotary_rows, rotary_dim)) != PA_OK)
    return st;
  if (mq < 0 || mk < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_query_len_bound/max_kv_len_bound: expected >= 0");
  if (kv->token_count == 0) return PA_OK;
  if ((st = check_kernel_support(params, kv, rt)) != PA_OK) return st;
  if ((st = check_norm_support(params)) != PA_OK) return st;
  if (!query) return fail(PA_ERR_INVALID_ARGUMENT, "query: expected non-NULL");
  if (!out) return fail(PA_ERR_INVALID_ARGUMENT, "out: expected non-NULL");
  if (!aligned16(query) || !aligned16(out))
    return fail(PA_ERR_INVALID_ARGUMENT, "query/out: expected 16-byte alignment");
  const Plan pl = make_plan(params, kv, rt, mq, mk);
  if ((st = check_plan(pl)) != PA_OK) return st;
  if (workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_INVALID_ARGUMENT, "workspace_bytes: expected >= %zu, got %zu",
                pl.ws_bytes, workspace_bytes);
  if (pl.ws_bytes > 0 && (!workspace || !aligned16(workspace)))
    return fail(PA_ERR_INVALID_ARGUMENT, "workspace: expected a 16-byte aligned pointer");

  const int D = params->head_size;
  const float scale = params->scale != 0.f ? params->scale : 1.0f / std::sqrt((float)D);
  const bool cap = params->softcap > 0.f;
  const float log2e = 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const pa::SeqLayout sl = layout(params, kv);

  pa::DecodeArgs d;
  d.s = sl;
  d.query = static_cast<const uint16_t*>(query);
  d.key_cache = static_cast<const uint16_t*>(kv->key_cache);
  d.value_cache = static_cast<const uint16_t*>(kv->value_cache);
  d.cos = static_cast<const uint16_t*>(cos_cache);
  d.sin = static_cast<const uint16_t*>(sin_cache);
  d.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  d.part_o = pl.listed ? reinterpret_cast<float*>(ws) : nullptr;
  d.part_ml = pl.listed ? reinterpret_cast<float*>(ws + pl.off_ml) : nullptr;
  d.entries = pl.listed ? reinterpret_cast<const pa::DecodeEntry*>(ws + pl.off_entries) : nullptr;
  d.entry_count = pl.listed ? reinterpret_cast<const int32_t*>(ws + pl.off_count) : nullptr;
  d.listed = pl.listed ? 1 : 0;
  d.rows = pl.rows;
  d.num_heads = params->num_heads;
  d.kv_heads = params->kv_num_heads;
  d.group = pl.g;
  d.head_chunks = pl.head_chunks;
  d.chunk_heads = pl.chunk_heads;
  d.token_mode = pl.token_mode ? 1 : 0;
  d.split_tokens = pl.split_tokens;
  d.max_splits = pl.max_splits;
  d.window = params->local_window_size;
  d.rotary_dim = params->do_rotary ? rotary_dim : 0;
  d.rotary_interleaved = params->rotary_interleaved;
  d.rotary_rows = params->do_rotary ? rotary_rows : 0;
  d.score_scale = scale * log2e;
  d.cap_in = cap ? scale / params->softcap : 0.f;
  d.cap_out = cap ? params->softcap * log2e : 0.f;
  d.use_softcap = cap ? 1 : 0;
  d.cache_dtype = params->cache_dtype;
  d.k_quant = params->k_quant_type;
  d.v_quant = params->v_quant_type;
  d.k_scale = kv->k_scale;
  d.v_scale = kv->v_scale;
  d.head_sink = static_cast<const uint16_t*>(params->head_sink);
  d.use_sink = params->head_sink || params->use_smooth_softmax ? 1 : 0;
  d.rotary_offset = params->do_rotary ? params->rotary_offset : 0;
  const bool latent = params->kv_cache_layout == PA_LAYOUT_LATENT;
  const int DV = effective_v_head_size(params);
  d.v_head_size = DV;
  // QK-Norm prologue (section 7.2): normalized queries staged in the
  // workspace; every attention kernel reads (and rotates) them from there
  if (pl.q_norm) {
    pa::QNormArgs qa;
    qa.in = static_cast<const uint16_t*>(query);
    qa.out = reinterpret_cast<uint16_t*>(ws + pl.off_qn);
    qa.rows = (int64_t)kv->token_count * params->num_heads;
    qa.head_size = D;
    qa.weight = static_cast<const uint16_t*>(params->q_norm_weight);
    qa.eps = norm_epsilon(params);
    StageScope scope(PA_STAGE_Q_NORM, s);
    if ((st = device_status(pa::launch_q_norm(qa, s), "QK-Norm prologue launch")) != PA_OK)
      return st;
    d.query = qa.out;
  }

  // prefill first, on the side stream when decode rows run beside it; the
  // side stream forks before the plan kernel, which only the decode needs
  // (pa_forward_noalloc creates nothing, not even the side stream: its launches
  // all go on the caller's stream, one after the other)
  const bool overlap = pl.prefill && pl.rows > 0 && !one_stream;
  hipStream_t ps = s;
  SideStream* side = nullptr;
  if (overlap) {
    if ((st = side_stream(s, &side)) != PA_OK) return st;
    hipError_t e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->st, side->fork, 0);
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "stream fork: %s", hipGetErrorString(e));
    ps = side->st;
  }
  // the join is queued whatever happens after the fork, so the caller's
  // stream never runs ahead of work queued on the side stream
  auto joined = [&](pa_status r) {
    if (!side) return r;
    hipError_t e = hipEventRecord(side->join, side->st);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
    side = nullptr;
    if (e != hipSuccess && r == PA_OK)
      return fail(PA_ERR_DEVICE, "stream join: %s", hipGetErrorString(e));
    return r;
  };
  if (pl.listed) {
    pa::PlanArgs pa_;
    pa_.s = sl;
    pa_.entries = reinterpret_cast<pa::DecodeEntry*>(ws + pl.off_entries);
    pa_.entry_count = reinterpret_cast<int32_t*>(ws + pl.off_count);
    pa_.row_split = reinterpret_cast<pa::RowSplit*>(ws + pl.off_rows);
    pa_.out = d.out;
    pa_.rows = pl.rows;
    pa_.token_mode = d.token_mode;
    pa_.split_tokens = pl.split_tokens;
    pa_.max_splits = pl.max_splits;
    pa_.window = params->local_window_size;
    pa_.row_width = params->num_heads * DV;
    StageScope scope(PA_STAGE_PLAN, s);
    if ((st = device_status(pa::launch_plan(pa_, s), "plan kernel launch")) != PA_OK)
      return joined(st);
  }
  if (pl.prefill) {
    pa::PrefillArgs f;
    f.s = sl;
    f.query = d.query;
    f.key_cache = d.key_cache;
    f.value_cache = d.value_cache;
    f.cos = d.cos;
    f.sin = d.sin;
    f.out = d.out;
    f.num_heads = params->num_heads;
    f.kv_heads = params->kv_num_heads;
    f.group = pl.g;
    f.window = params->local_window_size;
    f.rotary_dim = d.rotary_dim;
    f.rotary_interleaved = d.rotary_interleaved;
    f.rotary_rows = d.rotary_rows;
    f.tiles = pl.prefill_tiles;
    f.chunks = pl.prefill_chunks;
    f.piece_tiles = rt.prefill_pieces > 0 ? 0 : pa::kPrefillPieceTiles;
    f.part_o = pl.prefill_chunks > 1 ? reinterpret_cast<float*>(ws + pl.off_pf_o) : nullptr;
    f.part_ml = pl.prefill_chunks > 1 ? reinterpret_cast<float*>(ws + pl.off_pf_ml) : nullptr;
    f.score_scale = d.score_scale;
    f.cap_in2 = 2.0f * log2e * d.cap_in;
    f.cap_out = d.cap_out;
    f.use_softcap = d.use_softcap;
    f.rows16 = pl.prefill_kernel == 2;
    f.rows32 = pl.prefill_kernel == 3;
    f.tile_rows = pl.prefill_rows;
    f.key_tile = pl.prefill_kernel == 3 ? 32 : 64;
    f.pool32 = pool_fits_32bit(params, kv) ? 1 : 0;
    f.head_sink = d.head_sink;
    f.use_sink = d.use_sink;
    f.rotary_offset = d.rotary_offset;
    f.cache_dtype = d.cache_dtype;
    f.k_quant = d.k_quant;
    f.v_quant = d.v_quant;
    f.k_scale = d.k_scale;
    f.v_scale = d.v_scale;
    const dim3 grid(pl.prefill_tiles * pl.prefill_chunks + 1, params->kv_num_heads);
    {
      StageScope scope(PA_STAGE_PREFILL, ps);
      if ((st = device_status(pa::launch_prefill(f, D, grid, ps), "prefill kernel launch")) != PA_OK)
        return joined(st);
    }
    if (pl.prefill_chunks > 1) {
      StageScope scope(PA_STAGE_PREFILL_MERGE, ps);
      if ((st = device_status(pa::launch_prefill_merge(f, D, ps), "prefill merge launch")) != PA_OK)
        return joined(st);
    }
  }
  if (pl.rows > 0) {
    const int64_t hc = (int64_t)params->kv_num_heads * pl.head_chunks;
    int64_t wgs;
    if (pl.listed) {
      const int64_t bound = (int64_t)pl.rows * pl.max_splits * hc;
      // One workgroup per four possible items (those past the device list
      // exit at once) beside a prefill, so decode work spreads into the CUs
      // the prefill tiles free as they finish, and for long items (>= 256 KB
      // of K/V each), whose static round-robin over persistent workers leaves
      // a ragged tail that the hardware's dispatch evens out.  Short items
      // keep persistent workers: there extra workgroups cost more than they
      // balance.
      const int per_cu = latent ? pa::mla_workgroups_per_cu(d.use_softcap != 0)
                                : pa::decode_workgroups_per_cu(D, d.use_softcap != 0,
                                                               d.cache_dtype);
      const int64_t resident = (int64_t)per_cu * device_cus();
      const int64_t per_item = (bound + pa::kDecodeWaves - 1) / pa::kDecodeWaves;
      const int64_t row_bytes = latent ? 2 * D : 2 * 2 * D;   // K + V (or the latent row)
      const bool long_items = (int64_t)pl.split_tokens * row_bytes >= (256 << 10);
      wgs = overlap || long_items ? per_item : std::min<int64_t>(per_item, resident);
    } else {
      wgs = ((int64_t)pl.rows * hc + pa::kDecodeWaves - 1) / pa::kDecodeWaves;
    }
    {
      StageScope scope(PA_STAGE_DECODE, s);
      const int n = (int)std::max<int64_t>(wgs, 1);
      if ((st = device_status(latent ? pa::launch_mla(d, n, s) : pa::launch_decode(d, D, n, s),
                              "decode kernel launch")) != PA_OK)
        return joined(st);
    }
    if (pl.listed) {
      pa::MergeArgs mg;
      mg.row_split = reinterpret_cast<const pa::RowSplit*>(ws + pl.off_rows);
      mg.part_o = d.part_o;
      mg.part_ml = d.part_ml;
      mg.out = d.out;
      mg.rows = pl.rows;
      mg.num_heads = params->num_heads;
      mg.head_size = DV;
      mg.max_splits = pl.max_splits;
      mg.head_sink = d.head_sink;
      mg.use_sink = d.use_sink;
      StageScope scope(PA_STAGE_MERGE, s);
      if ((st = device_status(pa::launch_merge(mg, s), "merge kernel launch")) != PA_OK)
        return joined(st);
    }
  }
  return joined(PA_OK);
}

pa_status pa_forward(const pa_attn_params* params, const pa_paged_kv* kv, const void* query,
                     const void* cos_cache, const void* sin_cache, int32_t rotary_rows,
                     int32_t rotary_dim, int32_t mq, int32_t mk, void* workspace,
                     size_t workspace_bytes, void* out, void* stream) {
  const pa_routing rt = auto_routing();
  return forward_impl(params, kv, &rt, query, cos_cache, sin_cache, rotary_rows, rotary_dim, mq,
                      mk, workspace, workspace_bytes, out, stream);
}

pa_status pa_forward_noalloc(const pa_attn_params* params, const pa_paged_kv* kv,
                             const void* query, const void* cos_cache, const void* sin_cache,
                             int32_t rotary_rows, int32_t rotary_dim, int32_t mq, int32_t mk,
                             void* out, void* stream) {
  // validation and the plan first: an oversized plan is rejected before any
  // device call
  const pa_routing rt = auto_routing();
  size_t need = 0;
  pa_status st = workspace_bytes_impl(params, kv, &rt, mq, mk, &need);
  if (st != PA_OK) return st;
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_forward_noalloc: this plan needs %zu bytes of workspace, more than the "
                "%zu-byte scratch array (use pa_forward with a caller workspace)",
                need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (kv->token_count > 0) {
    if ((st = scratch_address(static_cast<hipStream_t>(stream), &ws)) != PA_OK) return st;
  }
  return forward_impl(params, kv, &rt, query, cos_cache, sin_cache, rotary_rows, rotary_dim, mq,
                      mk, ws, (size_t)PA_NOALLOC_SCRATCH_BYTES, out, stream, true);
}

pa_status pa_forward_routed(const pa_attn_params* params, const pa_paged_kv* kv,
                            const pa_routing* routing, const void* query,
                            const void* cos_cache, const void* sin_cache, int32_t rotary_rows,
                            int32_t rotary_dim, int32_t mq, int32_t mk, void* workspace,
                            size_t workspace_bytes, void* out, void* stream) {
  return forward_impl(params, kv, routing, query, cos_cache, sin_cache, rotary_rows, rotary_dim,
                      mq, mk, workspace, workspace_bytes, out, stream);
}

pa_status pa_bench_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  g_error.clear();
  if (!src || !sink) return fail(PA_ERR_INVALID_ARGUMENT, "src/sink: expected non-NULL");
  // whole 16 KB blocks: every lane's loads then stay inside the buffer
  if (bytes % 16384 != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "bytes: expected a multiple of 16384, got %zu", bytes);
  if (!aligned16(src)) return fail(PA_ERR_INVALID_ARGUMENT, "src: expected 16-byte alignment");
  if (bytes == 0) return PA_OK;
  return device_status(pa::launch_stream_read(src, (int64_t)bytes, sink,
                                              static_cast<hipStream_t>(stream)),
                       "stream read launch");
}

pa_status pa_timing_enable(int32_t max_launches) {
  g_error.clear();
  if (max_launches <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "max_launches: expected > 0, got %d", max_launches);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (hipEvent_t e : g_timing.events) (void)hipEventDestroy(e);
  g_timing.events.assign(2 * (size_t)max_launches, nullptr);
  g_timing.stage.assign(max_launches, -1);
  g_timing.used = 0;
  for (auto& e : g_timing.events) {
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      g_timing.enabled = false;
      return fail(PA_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorString(err));
    }
  }
  g_timing.enabled = true;
  return PA_OK;
}

pa_status pa_timing_disable(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (hipEvent_t e : g_timing.events) (void)hipEventDestroy(e);
  g_timing.events.clear();
  g_timing.stage.clear();
  g_timing.used = 0;
  g_timing.enabled = false;
  return PA_OK;
}

pa_status pa_timing_read(int32_t stage, double* total_ms, int32_t* launches) {
  g_error.clear();
  if (!total_ms || !launches)
    return fail(PA_ERR_INVALID_ARGUMENT, "total_ms/launches: expected non-NULL");
  if (stage < 0 || stage >= PA_NUM_STAGES)
    return fail(PA_ERR_INVALID_ARGUMENT, "stage: expected 0..%d, got %d", PA_NUM_STAGES - 1, stage);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  double tot = 0.0;
  int n = 0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    if (g_timing.stage[i] != stage) continue;
    hipError_t e = hipEventSynchronize(g_timing.events[2 * i + 1]);
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timing.events[2 * i], g_timing.events[2 * i + 1]);
    if (e != hipSuccess) return fail(PA_ERR_DEVICE, "hipEventElapsedTime: %s", hipGetErrorString(e));
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return PA_OK;
}

}  // extern "C"
