// Split-KV decode over the paged pool, its work-list planner and the
// log-sum-exp merge of splits.
//
// Work decomposition (GroupQueryAttention CPU Implementation Notes, "Flash
// Decoding": partials (m, l, o) per KV chunk, merged with exp(m_c - M)
// weights; PagedAttention -- CUDA Design Document, section 8.5 implementation
// note: each token's request is resolved on the device and pages are read in
// place; section 9.3.4 item 2: splits laid over the window-clamped interval
// [max(0, kv_len - W), kv_len); section 4.7: empty splits never reach the host).
//
// Each wave is an independent worker that owns one item: (row, kv head, head
// chunk, split).  It serves up to 16 query heads of the kv head's group at
// once, so every K/V byte of the split is read from HBM once.  Per tile of 32
// keys the wave computes, on the matrix cores,
//   S^T[key][head] = K[key][:] . Q[head][:]   (v_mfma_f32_16x16x32_f16)
//   O^T[d][head]  += V^T[d][key] . P^T[key][head]
// K and V load as whole key rows (1 KB per instruction), one tile ahead in
// registers, and are stored into the wave's own LDS tiles; the K operand is
// read back with 16-byte reads and the V^T operand with transposing reads.
// The score accumulator already has the B-operand layout of the PV product
// (keys ordered to match), so probabilities never leave registers.  A head's
// running max is shared by the four lanes that hold it with two cross-lane
// swaps per tile; the lane holding an output column also holds that head's
// max, so rescaling is local.  Scores are in log2 units (scale * log2 e
// folded in).
//
// Quantized caches (PagedAttention -- CUDA Design Document, section 8.5,
// phase 3): the rows are loaded as byte codes (half the bytes of fp16) and
// turned into fp16 on their way into the LDS tiles (int8 and e4m3fn values
// are all fp16 values, so the tiles hold the codes exactly).  The K scale is
// folded into the score scale (per tensor) or into Q (per channel), the V
// scale multiplies the output accumulator, so the products run on the codes.
#include <type_traits>

#include "decode_rows.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 units
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

// max / sum of a value and the one 16 (resp. 32) lanes away: one lane-swap
// instruction instead of a trip through the LDS crossbar
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// plan: one workgroup lists (row, split) entries; zeroes orphan token rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(const PlanArgs a) {
  __shared__ int s_wave[16];
  __shared__ int s_sum;
  __shared__ int s_first[1024];   // entry offset of each row of the chunk
  __shared__ RowInfo s_info[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  int total = 0;
  for (int r0 = 0; r0 < a.rows; r0 += 1024) {
    const int row = r0 + tid;
    int n = 0;
    if (row < a.rows) {
      RowInfo r;
      bool orphan;
      if (resolve_row(a.s, a.token_mode, row, a.window, a.split_tokens, a.max_splits, r, orphan)) {
        n = r.nsplit;
        s_info[tid] = r;
        // no key position to visit (the window starts past the table's
        // capacity): no item is listed, so the row is written here, as a
        // row with no admitted key
        if (n == 0)
          for (int i = 0; i < a.row_width; i += 8)
            store16(a.out + (int64_t)r.t * a.row_width + i, u32x4{0, 0, 0, 0});
      } else if (orphan) {
        for (int i = 0; i < a.row_width; i += 8)
          store16(a.out + (int64_t)row * a.row_width + i, u32x4{0, 0, 0, 0});
      }
      a.row_split[row] = RowSplit{n > 0 ? r.t : -1, n};
    }
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      int v = lane < 16 ? s_wave[lane] : 0;
      int sc = v;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int y = __shfl_up(sc, off, 64);
        if (lane >= off) sc += y;
      }
      if (lane < 16) s_wave[lane] = sc - v;
      if (lane == 15) s_sum = sc;
    }
    __syncthreads();
    // every thread writes entries: entry e of the chunk belongs to the last
    // row whose first entry is <= e (one row can own thousands of splits)
    s_first[tid] = s_wave[wv] + incl - n;
    __syncthreads();
    const int chunk_rows = min(1024, a.rows - r0);
    for (int e = tid; e < s_sum; e += 1024) {
      int lo = 0, hi = chunk_rows - 1;   // invariant: s_first[lo] <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_first[mid] <= e) lo = mid; else hi = mid - 1;
      }
      const RowInfo& r = s_info[lo];
      DecodeEntry en;
      en.row = r0 + lo;
      en.split = e - s_first[lo];
      en.k_lo = r.lo + en.split * a.split_tokens;
      en.k_hi = min(r.hi, en.k_lo + a.split_tokens);
      en.t = r.t;
      en.b = r.b;
      en.pos = r.pos;
      en.nsplit = r.nsplit;
      a.entries[total + e] = en;
    }
    total += s_sum;
    __syncthreads();
  }
  if (tid == 0 && a.entry_count) *a.entry_count = total;
}

// ---------------------------------------------------------------------------
// decode workers
// ---------------------------------------------------------------------------
template <int D>
struct DecodeCfg {
  static constexpr int KT = 32;          // keys per tile
  static constexpr int KS = D / 32;      // QK k-steps over the head dim
  static constexpr int DB = D / 16;      // 16-channel output blocks
  static constexpr int CH = D / 8;       // 16-byte chunks per key row
  static constexpr int RPI = 64 / CH;    // key rows per 1 KB load instruction
  static constexpr int NI = KT / RPI;    // load instructions per tile (K, and again V)
  static constexpr int KLD = D + 8;      // LDS row stride of K (halves): the 16 rows an
                                         // operand read touches sit 4 banks apart
  static constexpr int VLD = D + 16;     // LDS row stride of V: the 4 rows of a
                                         // transposing read sit 8 banks apart
  static constexpr int TBL = 256;        // block-table entries staged per segment
};

// One lane's 8 channels of a key row as loaded: fp16 (16 bytes) or 8 codes.
template <int CT>
using RawChunk = typename std::conditional<CT == kCacheF16, u32x4, u32x2>::type;

template <int CT>
__device__ __forceinline__ RawChunk<CT> load_chunk(const char* p) {
  return *reinterpret_cast<const RawChunk<CT>*>(p);
}

// The chunk as 8 fp16 values; rows that are not real keys become zeros.
template <int CT>
__device__ __forceinline__ u32x4 chunk_f16(RawChunk<CT> v, bool ok) {
  if (!ok) return u32x4{0, 0, 0, 0};
  if constexpr (CT == kCacheF16)
    return v;
  else
    return codes_to_f16<CT>(v);
}

// Whole key rows of one tile, K and V (RPI rows per instruction; lane l moves
// chunk l % CH of row l / CH: 1 KB of fp16, or 512 B of codes).  Bit i of the
// returned mask says whether the row of instruction i is a real key; the
// others read block 0 and are zeroed when stored, so nothing non-finite
// reaches the products.
template <int D, int CT>
__device__ __forceinline__ uint32_t load_tile(const char* kb, const char* vb,
                                              const int32_t* tbl, int first_bi, int shift,
                                              int64_t tok_stride, int k0, int seg_hi, int lane,
                                              RawChunk<CT> (&kr)[DecodeCfg<D>::NI],
                                              RawChunk<CT> (&vr)[DecodeCfg<D>::NI]) {
  using C = DecodeCfg<D>;
  constexpr int ES = CT == kCacheF16 ? 2 : 1;   // bytes per element
  const int bmask = (1 << shift) - 1;
  const int c = lane % C::CH;
  uint32_t okm = 0;
#pragma unroll
  for (int i = 0; i < C::NI; ++i) {
    const int key = k0 + i * C::RPI + lane / C::CH;
    const bool in = key < seg_hi;
    const int blk = tbl[in ? (key >> shift) - first_bi : 0];
    const bool ok = in && blk >= 0;
    okm |= (uint32_t)ok << i;
    const int64_t off =
        (((int64_t)(ok ? blk : 0) * (bmask + 1) + (key & bmask)) * tok_stride + 8 * c) * ES;
    kr[i] = load_chunk<CT>(kb + off);
    vr[i] = load_chunk<CT>(vb + off);
  }
  return okm;
}

template <int D, bool SOFTCAP, int CT>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D <= 64 ? 3 : D <= 128 ? 2 : 1)))
void decode_kernel(const DecodeArgs a) {
  using C = DecodeCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kDecodeWaves][C::KT * C::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kDecodeWaves][C::KT * C::VLD];
  __shared__ int32_t s_tbl[kDecodeWaves][C::TBL];

  // the wave index is uniform across the wave: saying so keeps every per-item
  // value (row, split, key range, pointers) and loop bound in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const SeqLayout& sl = a.s;
  const int HC = a.kv_heads * a.head_chunks;
  const int64_t HD = (int64_t)a.num_heads * D;
  const int total = a.listed ? (*a.entry_count) * HC : a.rows * HC;
  const int nworkers = gridDim.x * kDecodeWaves;
  uint16_t* kt = s_k[wave];
  uint16_t* vt = s_v[wave];
  int32_t* tbl = s_tbl[wave];
  const int shift = sl.block_shift;
  const int64_t tok_stride = (int64_t)a.kv_heads * D;
  constexpr int ES = CT == kCacheF16 ? 2 : 1;   // bytes per cache element
  // a per-tensor K scale joins the score scale (exact in the dot product:
  // the zero point is 0); a per-channel one is folded into Q below
  float score_scale = a.score_scale, cap_in = a.cap_in;
  bool k_per_channel = false;
  if constexpr (CT != kCacheF16) {
    if (a.k_quant == kQuantChannel) {
      k_per_channel = true;
    } else {
      const float ks = a.k_scale[0];
      score_scale *= ks;
      cap_in *= ks;
    }
  }

  // listed mode: the next item's entry is read while this item runs, and
  // (once this item's first tile loads are out) the block-table entries of
  // the next item's first segment, one per lane, when it spans <= 64 blocks
  DecodeEntry en_next;
  int32_t tbl_next = -1;
  bool tbl_next_ok = false;
  {
    const int first = blockIdx.x * kDecodeWaves + wave;
    if (a.listed && first < total) en_next = a.entries[first / HC];
  }
  for (int item = blockIdx.x * kDecodeWaves + wave; item < total; item += nworkers) {
    const int e = item / HC;
    const int kvhc = item - e * HC;
    const int kvh = kvhc / a.head_chunks;
    const int h0 = kvh * a.group + (kvhc - kvh * a.head_chunks) * a.chunk_heads;

    int row, split, k_lo, k_hi;
    RowInfo r;
    if (a.listed) {
      const DecodeEntry en = en_next;
      if (item + nworkers < total) en_next = a.entries[(item + nworkers) / HC];
      row = en.row;
      split = en.split;
      k_lo = en.k_lo;
      k_hi = en.k_hi;
      r.t = en.t;
      r.b = en.b;
      r.pos = en.pos;
      r.nsplit = en.nsplit;
    } else {
      row = e;
      split = 0;
      bool orphan;
      if (!resolve_row(sl, a.token_mode, row, a.window, a.split_tokens, a.max_splits, r, orphan)) {
        if (orphan && row < sl.tokens) {   // token owned by no request: zero
          for (int i = lane; i < a.chunk_heads * (D / 8); i += 64)
            store16(a.out + row * HD + (int64_t)h0 * D + 8 * i, u32x4{0, 0, 0, 0});
        }
        continue;
      }
      k_lo = r.lo;
      k_hi = r.nsplit > 0 ? min(r.hi, k_lo + a.split_tokens) : k_lo;
    }

    // Q as the B operand: lane (q, l16) holds head l16, channels 32ks + 8q + [0,8)
    const bool head_ok = l16 < a.chunk_heads;
    h8 qf[C::KS];
    {
      // all chunk loads first (one memory round trip), then the chunks that
      // RoPE rotates or a per-channel K scale multiplies
      const uint16_t* qrow = a.query + (int64_t)r.t * HD + (int64_t)(h0 + l16) * D;
      if (head_ok) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(load16(qrow + 8 * (4 * ks + q)));
      } else {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(u32x4{0, 0, 0, 0});
      }
      if (head_ok && (a.rotary_dim > 0 || k_per_channel)) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const int c = 4 * ks + q;
          const bool rot = chunk_rotated(c, a.rotary_offset, a.rotary_dim);
          if (rot || k_per_channel) {
            const int off = rot ? a.rotary_offset : 0;
            u32x4 v;
            __builtin_memcpy(&v, &qf[ks], 16);
            float rr[8];
            rotate_chunk(qrow + off, v, c - off / 8, r.pos, a.cos, a.sin, rot ? a.rotary_dim : 0,
                         a.rotary_interleaved, a.rotary_rows, rr);
            if (k_per_channel) {
              float ks8[8];
              channel_scales(a.k_scale, kQuantChannel, kvh, D, 8 * c, ks8);
#pragma unroll
              for (int e = 0; e < 8; ++e) rr[e] *= ks8[e];
            }
            qf[ks] = as_h8(pack8(rr));
          }
          __builtin_amdgcn_sched_barrier(0);   // one chunk at a time: keeps the prologue small
        }
      }
    }

    f4 acc[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    const char* kb = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * D * ES;
    const char* vb = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * D * ES;
    const int32_t* bt = sl.block_table + (int64_t)r.b * sl.maxblk;

    const bool have_next = a.listed && item + nworkers < total;
    const bool use_prefetch = tbl_next_ok;
    tbl_next_ok = false;
    for (int seg_lo = k_lo; seg_lo < k_hi;) {
      const int first_bi = seg_lo >> shift;
      const int seg_hi = min(k_hi, (first_bi + C::TBL) << shift);
      const int n_bi = ((seg_hi - 1) >> shift) - first_bi + 1;
      bool hole = false;
      if (use_prefetch && seg_lo == k_lo) {   // staged by the previous item (n_bi <= 64)
        if (lane < n_bi) {
          int v = tbl_next;
          if (v >= sl.num_blocks) v = -1;
          hole = v < 0;
          tbl[lane] = v;
        }
      } else {
        for (int i = lane; i < n_bi; i += 64) {
          const int bi = first_bi + i;
          int v = bi < sl.maxblk ? bt[bi] : -1;
          if (v >= sl.num_blocks) v = -1;
          hole |= v < 0;
          tbl[i] = v;
        }
      }
      const bool any_hole = __any(hole);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      const int ntile = (seg_hi - seg_lo + C::KT - 1) / C::KT;
      RawChunk<CT> kr[C::NI], vr[C::NI];
      uint32_t okm = load_tile<D, CT>(kb, vb, tbl, first_bi, shift, tok_stride, seg_lo, seg_hi,
                                      lane, kr, vr);
      if (have_next && seg_lo == k_lo) {
        // the next item's first-segment table, behind this tile's loads
        const int nlo = en_next.k_lo, nhi = en_next.k_hi;
        const int nfirst = nlo >> shift;
        const int nseg_hi = min(nhi, (nfirst + C::TBL) << shift);
        const int nn = nhi > nlo ? ((nseg_hi - 1) >> shift) - nfirst + 1 : 0;
        if (nn <= 64) {
          const int bi = nfirst + lane;
          tbl_next = lane < nn && bi < sl.maxblk
                         ? sl.block_table[(int64_t)en_next.b * sl.maxblk + bi]
                         : -1;
          tbl_next_ok = true;
        }
      }
      for (int it = 0; it < ntile; ++it) {
        const int k0 = seg_lo + it * C::KT;
        const bool more = it + 1 < ntile;

        // ---- this tile's rows into the wave's LDS tiles (zeros for masked
        // keys), then the next tile's loads go out into the freed registers ----
        {
          const int c = lane % C::CH;
#pragma unroll
          for (int i = 0; i < C::NI; ++i) {
            const int rw = i * C::RPI + lane / C::CH;
            const bool ok = (okm >> i) & 1u;
            store16(kt + rw * C::KLD + 8 * c, chunk_f16<CT>(kr[i], ok));
            store16(vt + rw * C::VLD + 8 * c, chunk_f16<CT>(vr[i], ok));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more)
          okm = load_tile<D, CT>(kb, vb, tbl, first_bi, shift, tok_stride, k0 + C::KT, seg_hi,
                                 lane, kr, vr);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- S^T = K . Q^T: two 16-key blocks ----
        f4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          s[sb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const h8 ka = *reinterpret_cast<const h8*>(kt + (16 * sb + l16) * C::KLD + 32 * ks + 8 * q);
            s[sb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[ks], s[sb], 0, 0, 0);
          }
        }

        // ---- scores (log2 units), mask, running max ----
        const bool edge = any_hole || k0 + C::KT > seg_hi;
        float x[8];
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float v = s[sb][rr];
            if constexpr (SOFTCAP)
              v = tanh_fast(v * cap_in) * a.cap_out;
            else
              v = v * score_scale;
            if (edge) {
              const int key = k0 + 16 * sb + 4 * q + rr;
              const bool ok = key < seg_hi && tbl[(key >> shift) - first_bi] >= 0;
              v = ok ? v : kNegInf;
            }
            x[4 * sb + rr] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = xor32_max(xor16_max(mx));
        // lazy rescale: keep the running max unless the tile exceeds it by more
        // than kRescaleSlack (probabilities then stay below 2^kRescaleSlack),
        // so most tiles skip touching the accumulators
        if (__any(mx > m + kRescaleSlack)) {
          const float mn = mx > m + kRescaleSlack ? mx : m;
          const float alpha = exp2_fast(m - (mn == kNegInf ? 0.f : mn));
          m = mn;
          lsum *= alpha;
#pragma unroll
          for (int i = 0; i < C::DB; ++i) acc[i] *= alpha;
        }
        const float mu = m == kNegInf ? 0.f : m;
        h8 pf;   // keys 4q + (0..3) of both 16-key blocks, in that order
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = exp2_fast(x[i] - mu);
          lsum += p;
          pf[i] = (_Float16)p;
        }

        // ---- O^T += V^T . P^T: the V^T operand by transposing LDS reads;
        // lane k of 16-lane group q points at 4 channels of key 4q + k / 4
        // (then 16 + 4q + k / 4), and lane i receives channel i of those four
        // keys -- the keys of this lane group's P values ----
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          v4s part[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
            part[sb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(
                    vt + (16 * sb + 4 * q + (l16 >> 2)) * C::VLD + 16 * db + 4 * (l16 & 3)));
          h8 va;
          __builtin_memcpy(&va, part, 16);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, acc[db], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      seg_lo = seg_hi;
      __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: lane (q, l16) holds head l16, channels 16db + 4q + [0,4) ----
    const float lt = xor32_sum(xor16_sum(lsum));
    if (head_ok) {
      const int h = h0 + l16;
      if constexpr (CT != kCacheF16) {
        // the V scale of channels 16db + 4q + [0, 4): output = scale * sum p code
        if (a.v_quant == kQuantChannel) {
          const float* vs = a.v_scale + (int64_t)kvh * D + 4 * q;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) acc[db] *= *reinterpret_cast<const f4*>(vs + 16 * db);
        } else {
          const float vs = a.v_scale[0];
#pragma unroll
          for (int db = 0; db < C::DB; ++db) acc[db] *= vs;
        }
      }
      if (r.nsplit <= 1) {
        const float den = sink_denominator(lt, m, a.use_sink, a.head_sink, h);
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        uint16_t* orow = a.out + (int64_t)r.t * HD + (int64_t)h * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          uint2 w;
          w.x = (uint32_t)f2h(acc[db][0] * inv) | ((uint32_t)f2h(acc[db][1] * inv) << 16);
          w.y = (uint32_t)f2h(acc[db][2] * inv) | ((uint32_t)f2h(acc[db][3] * inv) << 16);
          *reinterpret_cast<uint2*>(orow + 16 * db + 4 * q) = w;
        }
      } else {
        const int64_t pidx = ((int64_t)row * a.num_heads + h) * a.max_splits + split;
        float* po = a.part_o + pidx * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f4*>(po + 16 * db + 4 * q) = acc[db];
        if (q == 0) {
          a.part_ml[2 * pidx] = m;
          a.part_ml[2 * pidx + 1] = lt;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one workgroup per (row, group of heads) of rows with more than one
// split.  Thread (head, split group sg, 4-channel group dq) folds splits sg,
// sg + nsg, ... into a running (max, denominator, output) in one pass -- its
// loads go out eight splits at a time, ahead of the arithmetic -- and the
// split groups of each head are then combined pairwise in LDS (log2 nsg
// steps), each step rescaling both sides to the larger max
// (GroupQueryAttention CPU Implementation Notes, "Flash Decoding": partials
// weighted by exp(m_c - M)).  The host sizes nsg to the plan's split count
// and packs several heads into a workgroup when a head needs few threads.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 8;   // splits whose loads one thread issues together

__device__ __forceinline__ void merge_pair(float& M, float& den, f4& acc, float m2, float d2,
                                           f4 o2) {
  const float mn = fmaxf(M, m2);
  const float mu = mn == kNegInf ? 0.f : mn;
  const float a1 = exp2_fast(M - mu), a2 = exp2_fast(m2 - mu);
  acc = acc * a1 + o2 * a2;
  den = den * a1 + d2 * a2;
  M = mn;
}

template <int NT>
__global__ __launch_bounds__(NT) void merge_kernel(const MergeArgs a, const int hpw) {
  __shared__ f4 s_o[NT];
  __shared__ float2 s_md[NT];
  // workgroup id = row * head groups + head group: consecutive ids (one
  // row's head groups) land on different XCDs, so a long row's merge work
  // spreads over the chip
  const int ngroups = (a.num_heads + hpw - 1) / hpw;
  const int row = blockIdx.x / ngroups;
  const int hg = blockIdx.x - row * ngroups;
  const int tid = threadIdx.x;
  const RowSplit rs = a.row_split[row];
  if (rs.n <= 1) return;   // not a decode row, or the decode worker wrote it directly
  const int n = rs.n;
  const int D = a.head_size;
  const int nq = D >> 2;          // 4-channel groups (a power of two)
  const int per = NT / hpw;       // threads per head (a power-of-two multiple of nq)
  const int h = hg * hpw + tid / per;
  const int tl = tid % per;
  const int dq = tl % nq;
  const int sg = tl / nq;
  const int nsg = per / nq;
  const bool active = h < a.num_heads;
  float M = kNegInf, den = 0.f;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int64_t base = ((int64_t)row * a.num_heads + h) * a.max_splits;
    const float* po = a.part_o + base * D + 4 * dq;
    const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + base;
    for (int s0 = sg; s0 < n; s0 += nsg * kMergeBatch) {
      float2 ml[kMergeBatch];
      f4 o[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int s = s0 + i * nsg;
        ml[i] = s < n ? pml[s] : make_float2(kNegInf, 0.f);
        o[i] = s < n ? *reinterpret_cast<const f4*>(po + (int64_t)s * D)
                     : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) merge_pair(M, den, acc, ml[i].x, ml[i].y, o[i]);
    }
  }
  s_o[tid] = acc;
  s_md[tid] = make_float2(M, den);
  for (int half = nsg >> 1; half >= 1; half >>= 1) {
    __syncthreads();   // reads below touch groups [half, 2 half), writes [0, half)
    if (sg < half) {
      const float2 md = s_md[tid + half * nq];
      merge_pair(M, den, acc, md.x, md.y, s_o[tid + half * nq]);
      s_o[tid] = acc;
      s_md[tid] = make_float2(M, den);
    }
  }
  if (active && sg == 0) {
    den = sink_denominator(den, M, a.use_sink, a.head_sink, h);
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    uint2 w;
    w.x = (uint32_t)f2h(acc[0] * inv) | ((uint32_t)f2h(acc[1] * inv) << 16);
    w.y = (uint32_t)f2h(acc[2] * inv) | ((uint32_t)f2h(acc[3] * inv) << 16);
    *reinterpret_cast<uint2*>(a.out + (int64_t)rs.t * a.num_heads * D + (int64_t)h * D + 4 * dq) = w;
  }
}

template <int D, bool SOFTCAP, int CT>
int occupancy_wg() {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, SOFTCAP, CT>, 256, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    cached = n;
  }
  return cached;
}

template <int D, int CT>
int occupancy_of(bool softcap) {
  return softcap ? occupancy_wg<D, true, CT>() : occupancy_wg<D, false, CT>();
}

template <int D>
int occupancy_of_head(bool softcap, int cache_dtype) {
  switch (cache_dtype) {
    case kCacheI8: return occupancy_of<D, kCacheI8>(softcap);
    case kCacheF8: return occupancy_of<D, kCacheF8>(softcap);
    default: return occupancy_of<D, kCacheF16>(softcap);
  }
}

template <int D, int CT>
void launch_decode_cache(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t st) {
  if (a.use_softcap)
    launch_kernel(decode_kernel<D, true, CT>, grid, block, st, a);
  else
    launch_kernel(decode_kernel<D, false, CT>, grid, block, st, a);
}

template <int D>
void launch_decode_variant(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t st) {
  switch (a.cache_dtype) {
    case kCacheI8: launch_decode_cache<D, kCacheI8>(a, grid, block, st); break;
    case kCacheF8: launch_decode_cache<D, kCacheF8>(a, grid, block, st); break;
    default: launch_decode_cache<D, kCacheF16>(a, grid, block, st); break;
  }
}

}  // namespace

int decode_workgroups_per_cu(int head_size, bool softcap, int cache_dtype) {
  switch (head_size) {
    case 64: return occupancy_of_head<64>(softcap, cache_dtype);
    case 128: return occupancy_of_head<128>(softcap, cache_dtype);
    case 256: return occupancy_of_head<256>(softcap, cache_dtype);
    default: return 1;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  launch_kernel(plan_kernel, dim3(1), dim3(1024), st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int head_size, int workgroups, hipStream_t st) {
  const dim3 grid(workgroups), block(64 * kDecodeWaves);
  switch (head_size) {
    case 64: launch_decode_variant<64>(a, grid, block, st); break;
    case 128: launch_decode_variant<128>(a, grid, block, st); break;
    case 256: launch_decode_variant<256>(a, grid, block, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const int nq = a.head_size / 4;
  if (a.head_size % 4 || nq > 256 || (nq & (nq - 1)) || a.num_heads <= 0) return hipErrorInvalidValue;
  // split groups per head: enough that one batch of loads covers the plan's
  // splits (at most 1024 threads per head); heads share a workgroup of 256
  // threads when each needs fewer
  int nsg = 1;
  while (nsg * kMergeBatch < a.max_splits && nq * nsg < 1024) nsg *= 2;
  const int per = nq * nsg;
  const int nt = per > 256 ? 1024 : 256;
  int hpw = nt / per;
  while (hpw > 1 && hpw / 2 >= a.num_heads) hpw /= 2;   // no more heads than there are
  const int64_t wgs = (int64_t)a.rows * ((a.num_heads + hpw - 1) / hpw);
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (nt == 1024)
    launch_kernel(merge_kernel<1024>, grid, dim3(1024), st, a, hpw);
  else
    launch_kernel(merge_kernel<256>, grid, dim3(256), st, a, hpw);
  return hipGetLastError();
}

}  // namespace pa
