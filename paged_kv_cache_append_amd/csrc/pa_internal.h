// Internal launch interface between the host planner (pa_api.hip) and the
// gfx950 kernels (append.hip, decode.hip, prefill.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

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
};

// Decode kernel: one workgroup per (row, kv head [x head chunk], KV split).
// row = packed token (token mode) or request (request mode, q_len == 1 only).
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
  int32_t num_heads;
  int32_t kv_heads;
  int32_t group;                // H / Hkv
  int32_t head_chunks;          // group is covered in head_chunks chunks of G heads
  int32_t token_mode;           // 1: row = token; 0: row = request with q_len == 1
  int32_t split_tokens;         // KV tokens per split
  int32_t max_splits;           // S (grid z and workspace extent)
  int32_t window;               // -1 or W >= 1
  int32_t rotary_dim;
  int32_t rotary_interleaved;
  int32_t rotary_rows;
  float score_scale;            // scale * log2(e)           (no softcap)
  float cap_in;                 // scale / softcap            (softcap > 0)
  float cap_out;                // softcap * log2(e)          (softcap > 0)
  int32_t use_softcap;
};

// Split merge: one workgroup per (row), threads over (head, 8-channel chunk).
struct MergeArgs {
  SeqLayout s;
  const float* part_o;
  const float* part_ml;
  uint16_t* out;
  int32_t num_heads;
  int32_t head_size;
  int32_t token_mode;
  int32_t split_tokens;
  int32_t max_splits;
  int32_t window;
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
  int32_t tiles;                // grid.x - 1: tile slots; the last x zeroes orphan rows
  float score_scale;
  float cap_in;
  float cap_out;
  int32_t use_softcap;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int head_size, int g_chunk, dim3 grid,
                         hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st);

constexpr int kPrefillRows = 128;   // query rows (token x head) per prefill workgroup

}  // namespace pa
