// Split-KV decode over the paged pool, plus the log-sum-exp merge of splits.
//
// Work decomposition (GroupQueryAttention CPU Implementation Notes, "Flash
// Decoding": partials (m, l, o) per KV chunk, merged with exp(m_c - M)
// weights; PagedAttention -- CUDA Design Document, section 8.5 implementation
// note: the decode kernel resolves each token's request on the device and reads
// pages in place; section 9.3.4 item 2: splits laid over the window-clamped
// interval [max(0, kv_len - W), kv_len)).
//
// One workgroup (4 waves) owns (row, kv head, split) and serves all G query
// heads of the group, so each K/V byte of the split is read from HBM exactly
// once.  A token's D-channel row is spread over D/8 lanes, each holding one
// 16-byte chunk; a wave therefore covers 64/(D/8) tokens per load instruction
// and every token row is a contiguous 2*D-byte run of the NHD pool.  The lane
// keeps its G query chunks in registers (fp16 pairs for v_dot2_f32_f16), the
// per-token partial dot products are summed across the D/8 lanes with DPP row
// operations, and each lane group runs its own online softmax (running max,
// sum and unnormalised output for its 8 channels).  The block-table slice of
// the split is staged in LDS; K/V loads for the next group of tokens are
// issued before the current group is consumed.  At the end the lane groups and
// waves are merged (LDS), and the split either writes the fp16 row (single
// split) or its partial (m, l, o) for the merge kernel.  Scores are kept in
// log2 units (scale * log2 e folded in) so every exponential is one exp2.
#include "pa_device.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPT lanes; every lane of a group gets the total.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);            // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);            // quad_perm [2,3,0,1]
  if (LPT >= 8) v += dpp<0x141>(v);   // row_half_mirror: quad 0 <-> quad 1
  if (LPT >= 16) v += dpp<0x140>(v);  // row_mirror: half-row 0 <-> half-row 1
  if (LPT >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

struct RowInfo {
  int t, b, pos, lo, hi, nsplit;
};

// Resolve the query token a decode row stands for and the split layout of its
// admitted key interval [lo, hi).  Identical in the decode and merge kernels.
// Returns false when the row has no work for this kernel.
__device__ __forceinline__ bool resolve_row(const SeqLayout& s, int token_mode, int row,
                                            int window, int split_tokens, int max_splits,
                                            RowInfo& r, bool& orphan) {
  orphan = false;
  if (token_mode) {
    r.t = row;
    r.b = find_request(s.cum, s.batch, row);
    if (r.b < 0) {
      orphan = true;
      return false;
    }
    r.pos = s.past[r.b] + (row - s.cum[r.b]);
  } else {
    r.b = row;
    const int c0 = s.cum[row];
    if (s.cum[row + 1] - c0 != 1) return false;   // served by the prefill kernel
    r.t = c0;
    r.pos = s.past[row];
  }
  if (r.t < 0 || r.t >= s.tokens) return false;
  const int cap = s.maxblk << s.block_shift;
  r.hi = min(r.pos + 1, cap);
  r.lo = window > 0 ? max(0, r.pos + 1 - window) : 0;
  const int n = r.hi - r.lo;
  r.nsplit = n > 0 ? min((n + split_tokens - 1) / split_tokens, max_splits) : 0;
  return true;
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int LPT = D / 8;         // lanes per token row
  constexpr int TPW = 64 / LPT;      // tokens per wave per pass
  constexpr int NW = 4;              // waves per workgroup
  constexpr int U = 4;               // passes per load group
  constexpr int STEP = NW * TPW;     // tokens per pass over the workgroup
  constexpr int SEG = 256;           // block-table entries staged per segment

  __shared__ int32_t s_blk[SEG];
  __shared__ float s_o[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / LPT;
  const int c = lane % LPT;
  const int row = blockIdx.x;
  const int kvh = blockIdx.y / a.head_chunks;
  const int hc = blockIdx.y - kvh * a.head_chunks;
  const int split = blockIdx.z;
  const int h0 = kvh * a.group + hc * G;
  const int64_t HD = (int64_t)a.num_heads * D;
  const SeqLayout& sl = a.s;

  RowInfo r;
  bool orphan;
  if (!resolve_row(sl, a.token_mode, row, a.window, a.split_tokens, a.max_splits, r, orphan)) {
    if (orphan && split == 0 && row < sl.tokens) {   // token owned by no request: zero row
      for (int i = threadIdx.x; i < G * LPT; i += 256)
        store16(a.out + row * HD + (int64_t)(h0 + i / LPT) * D + 8 * (i % LPT), u32x4{0, 0, 0, 0});
    }
    return;
  }
  if (split >= max(r.nsplit, 1)) return;

  const int k_lo = r.lo + split * a.split_tokens;
  const int k_hi = r.nsplit > 0 ? min(r.hi, k_lo + a.split_tokens) : k_lo;

  // query chunks (rotated at the token's position, rounded to fp16)
  h2 q[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qrow = a.query + (int64_t)r.t * HD + (int64_t)(h0 + h) * D;
    u32x4 qv = load16(qrow + 8 * c);
    if (a.rotary_dim > 0 && 8 * c < a.rotary_dim) {
      float rr[8];
      rotate_chunk(qrow, qv, c, r.pos, a.cos, a.sin, a.rotary_dim, a.rotary_interleaved,
                   a.rotary_rows, rr);
      qv = pack8(rr);
    }
    __builtin_memcpy(&q[h][0], &qv, 16);
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }

  const int shift = sl.block_shift;
  const int bmask = (1 << shift) - 1;
  const int64_t tok_stride = (int64_t)a.kv_heads * D;
  const uint16_t* kbase = a.key_cache + (int64_t)kvh * D + 8 * c;
  const uint16_t* vbase = a.value_cache + (int64_t)kvh * D + 8 * c;
  const int32_t* bt = sl.block_table + (int64_t)r.b * sl.maxblk;
  const bool softcap = a.use_softcap != 0;

  for (int seg_lo = k_lo; seg_lo < k_hi;) {
    const int first_bi = seg_lo >> shift;
    const int seg_hi = min(k_hi, (first_bi + SEG) << shift);
    const int last_bi = (seg_hi - 1) >> shift;
    __syncthreads();
    if (threadIdx.x < SEG) {
      const int bi = first_bi + (int)threadIdx.x;
      int v = -1;
      if (bi <= last_bi && bi < sl.maxblk) {
        v = bt[bi];
        if (v >= sl.num_blocks) v = -1;
      }
      s_blk[threadIdx.x] = v;
    }
    __syncthreads();

    const int npass = (seg_hi - seg_lo + STEP - 1) / STEP;
    const int tok0 = seg_lo + wave * TPW + sub;

    u32x4 kc[U], vc[U];
    bool okc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tau = tok0 + u * STEP;
      okc[u] = false;
      kc[u] = vc[u] = u32x4{0, 0, 0, 0};
      if (tau < seg_hi) {
        const int blk = s_blk[(tau >> shift) - first_bi];
        if (blk >= 0) {
          const int64_t idx = ((int64_t)blk * (bmask + 1) + (tau & bmask)) * tok_stride;
          kc[u] = load16(kbase + idx);
          vc[u] = load16(vbase + idx);
          okc[u] = true;
        }
      }
    }

    for (int p0 = 0; p0 < npass; p0 += U) {
      // issue the next group's loads before consuming this one
      u32x4 kn[U], vn[U];
      bool okn[U];
      const bool more = p0 + U < npass;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        okn[u] = false;
        kn[u] = vn[u] = u32x4{0, 0, 0, 0};
        const int tau = tok0 + (p0 + U + u) * STEP;
        if (more && tau < seg_hi) {
          const int blk = s_blk[(tau >> shift) - first_bi];
          if (blk >= 0) {
            const int64_t idx = ((int64_t)blk * (bmask + 1) + (tau & bmask)) * tok_stride;
            kn[u] = load16(kbase + idx);
            vn[u] = load16(vbase + idx);
            okn[u] = true;
          }
        }
      }

      float sc[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const h8 kk = as_h8(kc[u]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h2 kp;
            kp[0] = kk[2 * i];
            kp[1] = kk[2 * i + 1];
            acc = __builtin_amdgcn_fdot2(q[h][i], kp, acc, false);
          }
          acc = group_sum<LPT>(acc);
          const float s = softcap ? tanh_fast(acc * a.cap_in) * a.cap_out : acc * a.score_scale;
          sc[u][h] = okc[u] ? s : kNegInf;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = sc[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
        const float mn = fmaxf(m[h], mx);
        const float mu = mn == kNegInf ? 0.f : mn;
        const float alpha = exp2_fast(m[h] - mu);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = exp2_fast(sc[u][h] - mu);
          l[h] += p;
          const h8 vv = as_h8(vc[u]);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = __builtin_fmaf(p, (float)vv[e], o[h][e]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kc[u] = kn[u];
        vc[u] = vn[u];
        okc[u] = okn[u];
      }
    }
    seg_lo = seg_hi;
  }

  // merge the lane groups of this wave (same channels, different tokens)
#pragma unroll
  for (int msk = LPT; msk < 64; msk <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], msk, 64);
      const float lo_ = __shfl_xor(l[h], msk, 64);
      const float mn = fmaxf(m[h], mo);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float fa = exp2_fast(m[h] - mu);
      const float fb = exp2_fast(mo - mu);
      l[h] = l[h] * fa + lo_ * fb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[h][e], msk, 64);
        o[h][e] = o[h][e] * fa + oo * fb;
      }
      m[h] = mn;
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][h][8 * c + e] = o[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // merge the waves; write the row (single split) or this split's partial
  if ((int)threadIdx.x < G * LPT) {
    const int h = threadIdx.x / LPT;
    const int cc = threadIdx.x % LPT;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    const float mu = M == kNegInf ? 0.f : M;
    float den = 0.f, num[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_fast(s_m[w][h] - mu);
      den += f * s_l[w][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] += f * s_o[w][h][8 * cc + e];
    }
    if (r.nsplit <= 1) {
      const float inv = den > 0.f ? 1.0f / den : 0.f;
      float res[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) res[e] = num[e] * inv;
      store16(a.out + (int64_t)r.t * HD + (int64_t)(h0 + h) * D + 8 * cc, pack8(res));
    } else {
      const int64_t pidx = ((int64_t)row * a.num_heads + h0 + h) * a.max_splits + split;
      float* po = a.part_o + pidx * D + 8 * cc;
#pragma unroll
      for (int e = 0; e < 8; ++e) po[e] = num[e];
      if (cc == 0) {
        a.part_ml[2 * pidx] = M;
        a.part_ml[2 * pidx + 1] = den;
      }
    }
  }
}

__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  const int row = blockIdx.x;
  RowInfo r;
  bool orphan;
  if (!resolve_row(a.s, a.token_mode, row, a.window, a.split_tokens, a.max_splits, r, orphan))
    return;
  if (r.nsplit <= 1) return;   // the decode kernel wrote this row directly
  const int D = a.head_size;
  const int chunks = D >> 3;
  const int items = a.num_heads * chunks;
  const int64_t HD = (int64_t)a.num_heads * D;
  for (int i = threadIdx.x; i < items; i += blockDim.x) {
    const int h = i / chunks;
    const int cc = i - h * chunks;
    const int64_t base = ((int64_t)row * a.num_heads + h) * a.max_splits;
    float M = kNegInf;
    for (int s = 0; s < r.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * (base + s)]);
    const float mu = M == kNegInf ? 0.f : M;
    float den = 0.f, num[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = 0.f;
    for (int s = 0; s < r.nsplit; ++s) {
      const float f = exp2_fast(a.part_ml[2 * (base + s)] - mu);
      den += f * a.part_ml[2 * (base + s) + 1];
      const float* po = a.part_o + (base + s) * D + 8 * cc;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] += f * po[e];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    float res[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = num[e] * inv;
    store16(a.out + (int64_t)r.t * HD + (int64_t)h * D + 8 * cc, pack8(res));
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int g_chunk, dim3 grid, hipStream_t st) {
  switch (g_chunk) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_size, int g_chunk, dim3 grid,
                         hipStream_t st) {
  switch (head_size) {
    case 64: return launch_decode_d<64>(a, g_chunk, grid, st);
    case 128: return launch_decode_d<128>(a, g_chunk, grid, st);
    case 256: return launch_decode_d<256>(a, g_chunk, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const MergeArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pa
