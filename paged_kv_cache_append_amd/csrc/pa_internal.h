// Internal launch interface between the host planner (pa_api.hip) and the
// gfx950 kernels (append.hip, decode.hip, prefill.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Cache element types and scale granularities (the values of the ABI enums).
constexpr int kCacheF16 = 0;    // fp16 elements
constexpr int kCacheI8 = 1;     // int8 codes
constexpr int kCacheF8 = 2;     // float8 e4m3fn codes
constexpr int kQuantNone = 0;
constexpr int kQuantTensor = 1; // one fp32 scale per cache
constexpr int kQuantChannel = 2;// one fp32 scale per (kv head, channel)

// Everything a kernel needs to resolve tokens, positions and pool slots on the
// device.  Lengths are always read on the device (PagedAttention -- CUDA
// Design Document, section 4.7: host values only select kernels and size
// launches).
struct SeqLayout {
  const int32_t* cum;          // [B + 1]
  const int32_t* past;         // [B]
  const int32_t* block_table;  // [B, maxblk]
  int32_t batch;               // B
  int32_t tokens;              // T
  int32_t maxblk;              // max_blocks_per_seq
  int32_t block_shift;         // log2(block_size)
  int64_t num_blocks;
};

struct AppendArgs {
  SeqLayout s;
  const int32_t* slot_mapping;   // null: slots derived from the block table
  const uint16_t* key;    // fp16 [T, Hkv*D]
  const uint16_t* value;  // fp16 [T, Hkv*D]
  uint16_t* key_cache;    // fp16 [NB, bs, Hkv, D]
  uint16_t* value_cache;
  const uint16_t* cos;    // fp16 [rows, rot/2] or null
  const uint16_t* sin;
  int32_t kv_heads;
  int32_t head_size;
  int32_t rotary_dim;     // 0 = off
  int32_t rotary_interleaved;
  int32_t rotary_rows;    // rows of cos/sin (positions beyond are not rotated)
  int32_t cache_dtype;    // kCache*: with codes the caches are byte arrays
  int32_t k_quant, v_quant;
  const float* k_scale;   // [1] or [Hkv, D]
  const float* v_scale;
  const uint16_t* k_norm; // QK-Norm weight of K (fp16 [D]) or null
  float norm_eps;
  int32_t rotary_offset;  // first rotated channel (multiple of 8)
};

// QK-Norm of the queries into a staging buffer (the prologue): rows of
// head_size channels, one weight vector shared by all heads.
struct QNormArgs {
  const uint16_t* in;     // fp16 [rows, D]
  uint16_t* out;          // fp16 [rows, D]
  int64_t rows;           // tokens * heads
  int32_t head_size;
  const uint16_t* weight; // fp16 [D]
  float eps;
};

// Decode work is a list of items (row, split) x (kv head, head chunk).  A row
// is a packed token (token mode) or a request with q_len == 1 (request mode);
// a split is a run of at most split_tokens keys of the row's admitted interval.
// With more than one possible split per row the list is built on the device
// by the plan kernel ("listed" mode); otherwise item = (row, split 0).
// One work-list entry: a (row, split) pair with what the decode workers need
// of the row already resolved (query token, request, position, split count)
// and the split's key interval [k_lo, k_hi).
struct DecodeEntry {
  int32_t row, split, k_lo, k_hi;
  int32_t t, b, pos, nsplit;
};

struct DecodeArgs {
  SeqLayout s;
  const uint16_t* query;        // fp16 [T, H*D]
  const uint16_t* key_cache;
  const uint16_t* value_cache;
  const uint16_t* cos;          // rotary tables or null
  const uint16_t* sin;
  uint16_t* out;                // fp16 [T, H*D]
  float* part_o;                // [rows, H, S, D]   unnormalised split outputs
  float* part_ml;               // [rows, H, S, 2]   (max in log2 units, sum)
  const DecodeEntry* entries;   // listed mode: work list
  const int32_t* entry_count;   // listed mode: number of entries
  int32_t listed;
  int32_t rows;
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;                // H / Hkv
  int32_t head_chunks;          // the group is covered in chunks of <= 16 heads
  int32_t chunk_heads;          // heads per chunk
  int32_t token_mode;           // 1: row = token; 0: row = request with q_len == 1
  int32_t split_tokens;         // KV tokens per split
  int32_t max_splits;           // S (workspace extent)
  int32_t window;               // -1 or W >= 1
  int32_t rotary_dim;
  int32_t rotary_interleaved;
  int32_t rotary_rows;
  float score_scale;            // scale * log2(e)           (no softcap)
  float cap_in;                 // scale / softcap            (softcap > 0)
  float cap_out;                // softcap * log2(e)          (softcap > 0)
  int32_t use_softcap;
  int32_t cache_dtype;          // kCache*: with codes key_cache/value_cache are byte arrays
  int32_t k_quant, v_quant;     // kQuant*
  const float* k_scale;         // [1] or [Hkv, D]
  const float* v_scale;
  const uint16_t* head_sink;    // fp16 [H] sink logits, or null (zero sinks)
  int32_t use_sink;             // 0: no sink term
  int32_t rotary_offset;        // first rotated channel (multiple of 8)
  int32_t v_head_size;          // output channels per head (latent: the V view of K)
};

// Plan kernel (one workgroup): lists (row, split) entries of every row with
// work, and zeroes output rows of tokens owned by no request (token mode).
// A decode row's output token and split count, as the plan resolved it
// (n = 0: not a decode row); the merge reads it instead of resolving again.
struct RowSplit {
  int32_t t, n;
};

struct PlanArgs {
  SeqLayout s;
  DecodeEntry* entries;
  int32_t* entry_count;
  RowSplit* row_split;          // [rows]
  uint16_t* out;
  int32_t rows;
  int32_t token_mode;
  int32_t split_tokens;
  int32_t max_splits;
  int32_t window;
  int32_t row_width;            // H * D elements of an output row
};

// Split merge: one workgroup per (row, head) of rows with more than one split.
struct MergeArgs {
  const RowSplit* row_split;    // written by the plan kernel
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  int32_t rows;
  int32_t num_heads;
  int32_t head_size;
  int32_t max_splits;
  const uint16_t* head_sink;    // as in DecodeArgs
  int32_t use_sink;
};

// Prefill kernel: one workgroup per (q tile of 128 rows, kv head).  Rows of a
// tile are (query token, head-in-group) pairs, token-major.
struct PrefillArgs {
  SeqLayout s;
  const uint16_t* query;
  const uint16_t* key_cache;
  const uint16_t* value_cache;
  const uint16_t* cos;
  const uint16_t* sin;
  uint16_t* out;
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;
  int32_t window;
  int32_t rotary_dim;
  int32_t rotary_interleaved;
  int32_t rotary_rows;
  int32_t tiles;                // tile slots; grid.x = tiles * chunks + 1 (the last x zeroes
                                // orphan rows)
  int32_t chunks;               // at most this many key-range pieces per tile
  int32_t piece_tiles;          // > 0: pieces of about this many 64-key tiles; 0: `chunks`
                                // equal pieces
  float* part_o;                // chunks > 1: [T, H, chunks, D] unnormalised outputs
  float* part_ml;               // [T, H, chunks, 2] (max in log2 units, sum)
  float score_scale;            // scale * log2(e)
  float cap_in2;                // 2 * log2(e) * scale / softcap  (tanh via exp2)
  float cap_out;                // softcap * log2(e)
  int32_t use_softcap;
  int32_t rows16;               // head_size 256: the 8-wave kernel (16 rows per wave)
  int32_t rows32;               // head_size 256, fp16 pools: the 8-wave kernel of 32 rows per
                                // wave (tiles of 256 rows and 32 keys)
  int32_t tile_rows;            // rows of a tile slot (kPrefillRows, or 2x for rows32)
  int32_t key_tile;             // keys per key tile (64, or 32 for rows32)
  int32_t pool32;               // each cache is smaller than 4 GiB (32-bit byte offsets)
  const uint16_t* head_sink;    // as in DecodeArgs
  int32_t use_sink;
  int32_t rotary_offset;
  int32_t cache_dtype;          // kCache*: with codes key_cache/value_cache are byte arrays
  int32_t k_quant, v_quant;     // kQuant*
  const float* k_scale;         // [1] or [Hkv, D]
  const float* v_scale;
};

// Kernel start/stop events of the launch being made on this thread (set by
// the host planner while per-kernel timing is on, else null).  With events,
// the launch goes through hipExtLaunchKernelGGL, which timestamps the
// dispatch itself instead of inserting separate event packets around it.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

template <typename... Args, typename... Params>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t st,
                          Args... args) {
  if (g_launch_events.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, g_launch_events.start, g_launch_events.stop,
                          0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// Launchers (return hipSuccess or the launch error).
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
hipError_t launch_q_norm(const QNormArgs& a, hipStream_t st);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int head_size, int workgroups, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
// resident decode workgroups per CU
int decode_workgroups_per_cu(int head_size, bool softcap, int cache_dtype);
hipError_t launch_prefill(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st);
hipError_t launch_prefill_merge(const PrefillArgs& a, int head_size, hipStream_t st);
// 8-wave prefill kernel of 16 rows per wave (head_size 256); grid as launch_prefill
hipError_t launch_prefill16(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st);
// 8-wave prefill kernel of 32 rows per wave (head_size 256, fp16 pools below 4 GiB)
hipError_t launch_prefill32(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st);
// latent attention (MLA): kv_num_heads 1, head_size 576, V = the leading 512
// channels of K; every row in token mode, items as for the decode kernel
hipError_t launch_mla(const DecodeArgs& a, int workgroups, hipStream_t st);
int mla_workgroups_per_cu(bool softcap);
// streaming read of `bytes` bytes (a multiple of 16 KB) for benchmarks
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t st);
constexpr int kMlaHeadSize = 576;
constexpr int kMlaVHeadSize = 512;
// byte offset of the latent kernel's zero rows (past the pool; a row read
// from there ends below 2^32): latent pools hold at most this many bytes
constexpr uint32_t kMlaZeroRow = 0xFFFFF000u;

constexpr int kPrefillRows = 128;   // query rows (token x head) per prefill workgroup
constexpr int kDecodeWaves = 4;     // independent decode workers per workgroup
constexpr int kDecodeMaxHeads = 16; // query heads served by one decode worker
constexpr int kDecodeMaxSplits = 2048;
constexpr int kPrefillChunks = 4;        // key-range pieces of a prefill tile in small batches
constexpr int kPrefillPieceTiles = 32;   // ... each about this many 64-key tiles
constexpr int kPrefillSplitItems = 1024; // ... used below this many (tile, kv head) items

}  // namespace pa
