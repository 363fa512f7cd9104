// Device helpers for the gfx950 kernels: fp16 packing, fast exp2 / tanh,
// wave reductions, and token -> request resolution.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its exponential form: tanh|x| = 1 - 2 / (exp(2|x|) + 1).
// Absolute error ~1e-7, which the softcap multiplies by at most `softcap`.
__device__ __forceinline__ float tanh_fast(float x) {
  float e = exp2_fast(fabsf(x) * (2.0f * kLog2e));
  float r = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return copysignf(r, x);
}

__device__ __forceinline__ float h2f(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f2h(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ __forceinline__ h8 as_h8(u32x4 v) {
  h8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Which request owns packed token t: the largest b with cum[b] <= t.
// Returns -1 when t >= cum[B] (PagedAttention -- CUDA Design Document,
// section 18.2: such tokens own nothing).
__device__ __forceinline__ int find_request(const int32_t* cum, int B, int t) {
  if (t >= cum[B]) return -1;
  int lo = 0, hi = B - 1;  // invariant: cum[lo] <= t (cum[0] = 0 by contract)
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Pool element offset of (block, offset-in-block, kv head, channel 0).
__device__ __forceinline__ int64_t slot_base(int64_t blk, int off, int kvh, int block_size,
                                             int kv_heads, int head_size) {
  return ((blk * block_size + off) * kv_heads + kvh) * (int64_t)head_size;
}

// ---- QK-Norm (PagedAttention -- CUDA Design Document, section 7.1) -------
// x[c] * w[c] / sqrt(mean_j x[j]^2 + eps) per head, the sum of squares in
// fp32; the result is rounded to fp16 (the staged fp16 rows of section 7.3).

// Sum over the `group` consecutive lanes (a power of two <= 64, aligned)
// that hold one head row; every lane of the group must be active.
__device__ __forceinline__ float group_sum(float v, int group) {
  for (int m = 1; m < group; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float sum_squares8(u32x4 x) {
  uint16_t h[8];
  __builtin_memcpy(h, &x, 16);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(h2f(h[e]), h2f(h[e]), ss);
  return ss;
}

// 1 / sqrt(sum of squares / head_size + eps), correctly rounded steps.
__device__ __forceinline__ float rms_inverse(float ss, int head_size, float eps) {
  return 1.0f / __builtin_sqrtf(ss / (float)head_size + eps);
}

// One fp16 value normalized: fp16(x * r * w).
__device__ __forceinline__ float norm_value(float x, float r, uint16_t w) {
  return (float)(_Float16)(x * r * h2f(w));
}

// Chunk [8c, 8c + 8) of a head row normalized with inverse rms r and weight w.
__device__ __forceinline__ u32x4 norm_chunk(u32x4 x, float r, const uint16_t* w, int c) {
  uint16_t h[8], wv[8];
  const u32x4 wc = load16(w + 8 * c);
  __builtin_memcpy(h, &x, 16);
  __builtin_memcpy(wv, &wc, 16);
  float f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = norm_value(h2f(h[e]), r, wv[e]);
  u32x4 out;
  uint16_t o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f2h(f[e]);
  __builtin_memcpy(&out, o, 16);
  return out;
}

// Rotary embedding of channels [8c, 8c+8) of one head row at position `pos`.
// `row` points at channel 0 of the head (global fp16), `own` holds the chunk.
// With a norm weight `nw` (QK-Norm before RoPE) the row in memory is the
// raw one: partner values read from it are normalized with (nr, nw) first,
// and `own` must already be normalized.
// Pairs are (i, i + r/2) (rotate-half) or (2i, 2i+1) (interleaved) with angle
// index i; first' = x*cos - y*sin, second' = y*cos + x*sin; channels >= r pass
// through.  Both products of fp16 values are exact in fp32, so the fused
// multiply-add below rounds the exact result once -- the stored key is then
// fp16(fp32(exact)).  Positions outside the table are not rotated (memory
// safety for out-of-contract device lengths).
// Whether chunk c (channels [8c, 8c + 8)) of a head row meets the rotary
// window [off, off + rot) (PagedAttention -- CUDA Design Document, section
// 12.5: RoPE may cover a suffix; off is a multiple of 8).  Callers then pass
// the row from channel off and the chunk index c - off / 8.
__device__ __forceinline__ bool chunk_rotated(int c, int off, int rot) {
  return rot > 0 && 8 * c >= off && 8 * c < off + rot;
}

__device__ __forceinline__ float rot_pair(float x, float y, float cs, float sn, bool second) {
  const float ys = y * sn;  // exact
  return second ? __builtin_fmaf(x, cs, ys) : __builtin_fmaf(x, cs, -ys);
}

__device__ __forceinline__ void rotate_chunk(const uint16_t* row, u32x4 own, int c, int pos,
                                             const uint16_t* cos_t, const uint16_t* sin_t,
                                             int rot, int interleaved, int rot_rows,
                                             float out[8], float nr = 0.f,
                                             const uint16_t* nw = nullptr) {
  uint16_t x16[8];
  __builtin_memcpy(x16, &own, 16);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = h2f(x16[e]);
  const int d0 = 8 * c;
  if (pos < 0 || pos >= rot_rows || d0 >= rot) return;
  const int half = rot >> 1;
  const int64_t tb = (int64_t)pos * half;
  if (!interleaved && (half & 7) == 0) {
    // the chunk lies in one half: partner chunk and 8 consecutive angles
    const bool second = d0 >= half;
    const int i0 = second ? d0 - half : d0;
    uint16_t y16[8], c16[8], s16[8];
    const int pc = (second ? d0 - half : d0 + half) >> 3;
    u32x4 pv = load16(row + 8 * pc);
    if (nw) pv = norm_chunk(pv, nr, nw, pc);
    const u32x4 cv = load16(cos_t + tb + i0);
    const u32x4 sv = load16(sin_t + tb + i0);
    __builtin_memcpy(y16, &pv, 16);
    __builtin_memcpy(c16, &cv, 16);
    __builtin_memcpy(s16, &sv, 16);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = rot_pair(h2f(x16[e]), h2f(y16[e]), h2f(c16[e]), h2f(s16[e]), second);
  } else if (interleaved && (half & 7) == 0) {
    // pairs (2i, 2i+1) inside the chunk: 4 consecutive angles
    uint16_t c16[4], s16[4];
    const uint2 cv = *reinterpret_cast<const uint2*>(cos_t + tb + (d0 >> 1));
    const uint2 sv = *reinterpret_cast<const uint2*>(sin_t + tb + (d0 >> 1));
    __builtin_memcpy(c16, &cv, 8);
    __builtin_memcpy(s16, &sv, 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      out[e] = rot_pair(h2f(x16[e]), h2f(x16[e ^ 1]), h2f(c16[e >> 1]), h2f(s16[e >> 1]),
                        (e & 1) != 0);
  } else {
    // general layout: one channel at a time (kept rolled to stay small)
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      if (d >= rot) break;
      const bool second = interleaved ? (d & 1) != 0 : d >= half;
      const int i = interleaved ? (d >> 1) : (second ? d - half : d);
      const int partner = interleaved ? (d ^ 1) : (second ? d - half : d + half);
      const float y = nw ? norm_value(h2f(row[partner]), nr, nw[partner]) : h2f(row[partner]);
      out[e] = rot_pair(h2f(x16[e]), y, h2f(cos_t[tb + i]), h2f(sin_t[tb + i]), second);
    }
  }
}

__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  uint16_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = f2h(f[e]);
  u32x4 r;
  __builtin_memcpy(&r, h, 16);
  return r;
}

// ---- quantized caches (PagedAttention -- CUDA Design Document, section 8):
// codes are stored with zero point 0, value = code * scale -------------------

// Eight int8 codes -> eight fp16 values (exact).  code + 128 becomes the low
// mantissa byte of 1024.0 (0x64xx), then one packed subtraction of 1152.
__device__ __forceinline__ u32x4 int8x8_to_f16(u32x2 c) {
  const uint32_t x0 = c[0] ^ 0x80808080u, x1 = c[1] ^ 0x80808080u;
  const uint32_t w[4] = {__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u),
                         __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h2 v;
    __builtin_memcpy(&v, &w[i], 4);
    v -= h2{(_Float16)1152.0f, (_Float16)1152.0f};
    __builtin_memcpy(&r[i], &v, 4);
  }
  return u32x4{r[0], r[1], r[2], r[3]};
}

// Eight float8 e4m3fn codes -> eight fp16 values (every e4m3fn value, NaN
// included, is an fp16 value: exact), two codes per conversion.
__device__ __forceinline__ u32x4 fp8x8_to_f16(u32x2 c) {
  const h2 v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[0], 1.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[0], 1.0f, true),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[1], 1.0f, false),
                   __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[1], 1.0f, true)};
  u32x4 r;
  __builtin_memcpy(&r, v, 16);
  return r;
}

template <int CT>
__device__ __forceinline__ u32x4 codes_to_f16(u32x2 c) {
  if constexpr (CT == kCacheI8)
    return int8x8_to_f16(c);
  else
    return fp8x8_to_f16(c);
}

// The fp32 scale of channels [d0, d0 + 8) of kv head kvh.
__device__ __forceinline__ void channel_scales(const float* scale, int quant, int kvh,
                                               int head_size, int d0, float s[8]) {
  if (quant == kQuantChannel) {
    const float* p = scale + (int64_t)kvh * head_size + d0;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
  } else {
    const float v = scale[0];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = v;
  }
}

// Codes of eight fp16 values: saturate(round-half-even(fp32(x) / s)), one
// correctly rounded fp32 division per value.  int8 saturates to [-128, 127];
// e4m3fn to +-448, after which the hardware conversion rounds to nearest even.
__device__ __forceinline__ u32x2 quantize8(u32x4 x16, int cache_dtype, const float s[8]) {
  uint16_t h[8];
  __builtin_memcpy(h, &x16, 16);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = h2f(h[e]) / s[e];
  u32x2 r;
  if (cache_dtype == kCacheI8) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      b[e] = (uint32_t)(int32_t)fminf(fmaxf(__builtin_rintf(y[e]), -128.0f), 127.0f) & 0xFFu;
    r[0] = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    r[1] = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(y[e], -448.0f), 448.0f);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w], y[4 * w + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w + 2], y[4 * w + 3], v, true);
      r[w] = (uint32_t)v;
    }
  }
  return r;
}

// ---- attention sink (PagedAttention -- CUDA Design Document, section 6.1) --
// The head's sink logit s joins the softmax denominator only.  Scores are
// kept as 2^(x log2 e - m) with running max m (log2 units) and sum l, so the
// denominator becomes l + 2^(s log2 e - m).  A row with no key at all
// (m = -inf, l = 0, output 0) keeps l, so a sink of -inf cannot make it NaN.
__device__ __forceinline__ float sink_denominator(float l, float m, int use_sink,
                                                  const uint16_t* sink, int h) {
  if (!use_sink || m == -__builtin_huge_valf()) return l;
  const float s = sink ? h2f(sink[h]) : 0.f;   // no array: smooth softmax (s = 0)
  return l + exp2_fast(s * kLog2e - m);
}

template <int W>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace pa
