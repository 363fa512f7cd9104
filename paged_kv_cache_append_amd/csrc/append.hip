// KV append: scatter every new token's K/V row into its pool slot
// (PagedAttention -- CUDA Design Document, section 5.1 "derived write slot",
// section 5.2 explicit slot_mapping; Design: WebGPU PagedAttention, section 5
// Phase 1 item 3 for the one-lane-per-vector dispatch over token_count *
// kv_hidden).
//
// One lane moves one 16-byte chunk (8 channels) of one (token, kv head) for
// both K and V.  Lanes of a wave cover consecutive chunks of a token row, so
// the NHD pool layout turns every token into one contiguous Hkv*D*2-byte run:
// fully coalesced reads and writes.  The owning request is found by binary
// search over cumulative_sequence_length (same-address loads across the
// wave, served by the cache); tokens at or past cum[B] own nothing (the
// out-of-bounds defect of section 18.2 cannot occur).  With an explicit slot
// mapping the slot is read, not derived (-1: no write); the request is then
// only looked up for the rotary position.
//
// QK-Norm (section 7.2: normalize, then RoPE, then write): the lanes of one
// (token, kv head) row are D/8 consecutive, aligned lanes of a wave; they sum
// their squares across the group before any lane leaves for lack of a slot,
// normalize their own chunk, and normalize the partner chunk RoPE reads.
//
// Quantized caches (section 8.4, write path): the lane turns its 8 channels
// -- after rotary, as fp16, exactly the values an fp16 cache would hold --
// into 8 byte codes with the channels' fp32 scales and stores 8 bytes.
#include "pa_device.h"

namespace pa {

__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  const int chunks = a.head_size >> 3;
  const int64_t per_tok = (int64_t)a.kv_heads * chunks;
  const int64_t items = (int64_t)a.s.tokens * per_tok;
  const int bs = 1 << a.s.block_shift;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
    const int t = (int)(it / per_tok);
    const int rem = (int)(it - (int64_t)t * per_tok);
    const int kvh = rem / chunks;
    const int c = rem - kvh * chunks;
    const int64_t src_row = (int64_t)t * a.kv_heads * a.head_size + (int64_t)kvh * a.head_size;
    u32x4 k = load16(a.key + src_row + 8 * c);
    // V goes out with K, ahead of the slot lookup's dependent loads (a latent
    // cache, section 12.2, has no V: V is a view of K)
    const u32x4 v = a.value ? load16(a.value + src_row + 8 * c) : u32x4{0, 0, 0, 0};
    float nr = 0.f;
    if (a.k_norm) {
      nr = rms_inverse(group_sum(sum_squares8(k), chunks), a.head_size, a.norm_eps);
      k = norm_chunk(k, nr, a.k_norm, c);
    }
    int64_t blk;
    int off, pos = -1;
    if (a.slot_mapping) {
      if (t >= a.s.cum[a.s.batch]) continue;          // owned by no request
      const int32_t sm = a.slot_mapping[t];
      if (sm < 0 || (int64_t)sm >= (a.s.num_blocks << a.s.block_shift)) continue;   // -1: no write
      blk = sm >> a.s.block_shift;
      off = sm & (bs - 1);
      if (chunk_rotated(c, a.rotary_offset, a.rotary_dim)) {
        const int b = find_request(a.s.cum, a.s.batch, t);
        pos = a.s.past[b] + (t - a.s.cum[b]);
      }
    } else {
      const int b = find_request(a.s.cum, a.s.batch, t);
      if (b < 0) continue;
      pos = a.s.past[b] + (t - a.s.cum[b]);
      if (pos < 0) continue;
      const int bi = pos >> a.s.block_shift;
      if (bi >= a.s.maxblk) continue;
      blk = a.s.block_table[(int64_t)b * a.s.maxblk + bi];
      if (blk < 0 || blk >= a.s.num_blocks) continue;  // unmapped: nothing to write
      off = pos & (bs - 1);
    }
    const int64_t dst = slot_base(blk, off, kvh, bs, a.kv_heads, a.head_size) + 8 * c;
    if (chunk_rotated(c, a.rotary_offset, a.rotary_dim)) {
      const int off = a.rotary_offset;
      float r[8];
      rotate_chunk(a.key + src_row + off, k, c - off / 8, pos, a.cos, a.sin, a.rotary_dim,
                   a.rotary_interleaved, a.rotary_rows, r, nr, a.k_norm ? a.k_norm + off : nullptr);
      k = pack8(r);
    }
    if (a.cache_dtype == kCacheF16) {
      if (a.value_cache) store16(a.value_cache + dst, v);
      store16(a.key_cache + dst, k);
    } else {
      float sk[8], sv[8];
      channel_scales(a.k_scale, a.k_quant, kvh, a.head_size, 8 * c, sk);
      channel_scales(a.v_scale, a.v_quant, kvh, a.head_size, 8 * c, sv);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.value_cache) + dst) =
          quantize8(v, a.cache_dtype, sv);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.key_cache) + dst) =
          quantize8(k, a.cache_dtype, sk);
    }
  }
}

// The prologue of a forward with QK-Norm (section 7.2-7.3): every query head
// row normalized into an fp16 staging buffer, which the attention kernels
// then read (and rotate) in place of the query.  One lane per 8 channels;
// the D/8 lanes of a row are consecutive and aligned.
__global__ __launch_bounds__(256) void q_norm_kernel(const QNormArgs a) {
  const int chunks = a.head_size >> 3;
  const int64_t items = a.rows * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
    const int64_t row = it / chunks;
    const int c = (int)(it - row * chunks);
    const u32x4 x = load16(a.in + row * a.head_size + 8 * c);
    const float r = rms_inverse(group_sum(sum_squares8(x), chunks), a.head_size, a.eps);
    store16(a.out + row * a.head_size + 8 * c, norm_chunk(x, r, a.weight, c));
  }
}

hipError_t launch_q_norm(const QNormArgs& a, hipStream_t st) {
  const int64_t items = a.rows * (a.head_size >> 3);
  if (items == 0) return hipSuccess;
  int64_t blocks = (items + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  launch_kernel(q_norm_kernel, dim3((unsigned)blocks), dim3(256), st, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.s.tokens * a.kv_heads * (a.head_size >> 3);
  if (items == 0) return hipSuccess;
  int64_t blocks = (items + 255) / 256;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  launch_kernel(append_kernel, dim3((unsigned)blocks), dim3(256), st, a);
  return hipGetLastError();
}

}  // namespace pa
