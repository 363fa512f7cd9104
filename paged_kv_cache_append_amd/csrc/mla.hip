// Latent attention (MLA) over the paged cache: absorbed-form multi-query
// attention with a wide head (PagedAttention -- CUDA Design Document, section
// 12.2: one cache, kv_num_heads = 1, V = the leading v_head_size channels of
// K; section 12.5: RoPE on the channel suffix [rotary_offset, +rotary_dim)).
//
// A cache row is 576 fp16 channels: 512 latent + 64 rotary.  The work
// decomposition is the decode kernel's (decode.hip): persistent waves take
// items (row, head chunk of up to 16 query heads, key split) from the same
// device-built list, and splits are merged by the same merge kernel (with
// 512-channel partials).  Every query token is a row (token mode), so decode,
// chunked prefill and prefill all take this path, as the pages' own latent
// reference does (section 13).
//
// RoPE may only cover channels past the V view (rotary_offset >= 512):
// rotating latent channels would rotate V as well.
//
// Per tile of 32 keys a wave
//   - writes the rows (36 KB), which it loaded into registers while the
//     previous tile was computed, into its own LDS tile, and issues the loads
//     of the next tile (one wave per SIMD, so the Q fragments, the
//     512-channel accumulator and the 144 registers of a staged tile fit):
//     one 1 KB load per row for channels 0..511 (rows 1056 B apart in LDS,
//     32 mod 64), and one per 8 rows for the rotary channels 512..575 (a
//     128-byte-per-row tail region whose 16-byte slots are XOR-swizzled by
//     row).  Keys that are masked or past the split read offsets beyond the
//     buffer's end, which load zeros.  (Direct loads into LDS, with the next
//     copy issued once the tile's last read returned, measured 3.5 % slower
//     on a 16-head batch: a wave then had no load in flight while it
//     computed.);
//   - computes S^T = K . Q^T on the matrix cores (18 k-steps of
//     v_mfma_f32_16x16x32_f16 per 16-key block, Q fragments in registers);
//   - runs the online softmax in registers (log2 units);
//   - computes O^T += V^T . P^T with V^T read from the SAME tile by
//     transposing reads (ds_read_b64_tr_b16): V is never loaded separately.
// The head chunks of one (row, split) are consecutive items, taken by waves
// of one workgroup, so the rows they share come from L2 after the first read.
//
// With 64 or more heads (four head chunks or more) a workgroup of 8 waves
// takes four head chunks of the same (row, split) and shares one
// double-buffered LDS tile pair; the two waves of a pair split a chunk's
// products (QK over channel halves, PV over output halves), so each holds
// half the registers and two waves share every SIMD (mla_pair_kernel).  A
// tile is copied once per 64 heads instead of once per 16.
#include <type_traits>

#include "decode_rows.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 units
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

// LDS operand reads in flight ahead of the products that use them
constexpr int kAheadK = 4;
constexpr int kAheadV = 4;

struct MlaCfg {
  static constexpr int D = kMlaHeadSize;     // 576: latent 512 + rotary 64
  static constexpr int DV = kMlaVHeadSize;   // 512: the V view of a row
  static constexpr int KT = 32;              // keys per tile
  static constexpr int KS = D / 32;          // 18 QK k-steps
  static constexpr int DB = DV / 16;         // 32 output blocks of 16 channels
  static constexpr int MAIN = 1024 + 32;     // bytes per row of channels 0..511
  static constexpr int TAIL = 128;           // bytes per row of channels 512..575
  static constexpr int TILE = KT * (MAIN + TAIL);   // 37888 bytes of LDS per wave
  static constexpr int TBL = 256;            // block-table entries staged per segment
  static constexpr int WAVES = 4;
};

__device__ __forceinline__ float lane_max16(float v) {
  const auto r =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_max32(float v) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_sum16(float v) {
  const auto r =
      __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_sum32(float v) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tail region: row r's rotary chunk c (channels 512 + 8 c, c < 8) sits in
// 16-byte slot (c ^ (r & 7)) of the row's 128 bytes.
__device__ __forceinline__ int tail_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Byte offset in the pool of channel 0 of key `key`, or kMlaZeroRow (a row
// past the buffer's end, which loads zeros) when the key is outside the split
// or unmapped.  The host keeps the pool at or below kMlaZeroRow bytes.
__device__ __forceinline__ uint32_t mla_row_offset(const int32_t* tbl, int first_bi, int shift,
                                                   int key, int seg_hi) {
  const bool in = key < seg_hi;
  const int blk = tbl[in ? (key >> shift) - first_bi : 0];
  if (!in || blk < 0) return kMlaZeroRow;
  const uint32_t row = ((uint32_t)blk << shift) | (uint32_t)(key & ((1 << shift) - 1));
  return row * (uint32_t)(2 * MlaCfg::D);
}

// Copy rows 8 g0 .. 8 (g0 + NG) - 1 of the tile of keys k0 .. k0 + 31 into
// an LDS tile (main rows, then their tail): 9 NG instructions.  Lane l looks
// up the offset of row 8 g0 + l % (8 NG) (one table read per lane, in
// parallel); each row's offset is then broadcast to the wave.
template <int NG>
__device__ __forceinline__ void mla_copy_rows(__amdgpu_buffer_rsrc_t srd, char* tile,
                                              const int32_t* tbl, int first_bi, int shift,
                                              int k0, int seg_hi, int lane, int g0) {
  using C = MlaCfg;
  const uint32_t mine =
      mla_row_offset(tbl, first_bi, shift, k0 + 8 * g0 + (lane & (8 * NG - 1)), seg_hi);
#pragma unroll
  for (int r = 0; r < 8 * NG; ++r) {
    const uint32_t base = __builtin_amdgcn_readlane(mine, r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        srd, (__attribute__((address_space(3))) void*)(tile + (8 * g0 + r) * C::MAIN), 16,
        base + 16 * lane, 0, 0, 0);
  }
  // tail: lane l fills slot l of 8 rows; slot s of row r holds chunk s ^ (r & 7)
  const int rr = lane >> 3, cc = (lane & 7) ^ (rr & 7);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t base = (uint32_t)__shfl((int)mine, 8 * g + rr, 64);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        srd,
        (__attribute__((address_space(3))) void*)(tile + C::KT * C::MAIN +
                                                  8 * (g0 + g) * C::TAIL),
        16, base + 2 * (C::DV + 8 * cc), 0, 0, 0);
  }
}

// Per-wave mode (fewer than four head chunks): each wave an independent
// worker with its own LDS tile.
template <bool SOFTCAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void mla_kernel(const DecodeArgs a) {
  using C = MlaCfg;
  __shared__ __attribute__((aligned(16))) char s_k[C::WAVES][C::TILE];
  __shared__ int32_t s_tbl[C::WAVES][C::TBL];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const SeqLayout& sl = a.s;
  const int HC = a.head_chunks;                       // one kv head
  const int64_t HQ = (int64_t)a.num_heads * C::D;     // query row width
  const int64_t HO = (int64_t)a.num_heads * C::DV;    // output row width
  const int HG = HC;
  const int total = a.listed ? (*a.entry_count) * HG : a.rows * HG;
  const int nworkers = gridDim.x * C::WAVES;
  int32_t* tbl = s_tbl[wave];
  const int shift = sl.block_shift;
  // the pool as a buffer: 32-bit byte offsets (the host checks it is < 4 GiB)
  const int64_t pool_bytes = (sl.num_blocks << shift) * (int64_t)(2 * C::D);
  const __amdgpu_buffer_rsrc_t srd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.key_cache, (short)0, (int)(uint32_t)min(pool_bytes, (int64_t)0xFFFFFFFF),
      0x00020000);

  for (int item = blockIdx.x * C::WAVES + wave; item < total; item += nworkers) {
    const int e = item / HG;
    const int hc = item - e * HG;
    const int h0 = hc * a.chunk_heads;

    int row, split, k_lo, k_hi;
    RowInfo r;
    if (a.listed) {
      const DecodeEntry en = a.entries[e];
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
      if (!resolve_row(sl, 1, row, a.window, a.split_tokens, a.max_splits, r, orphan)) {
        if (orphan && row < sl.tokens) {   // token owned by no request: zero
          for (int i = lane; i < a.chunk_heads * (C::DV / 8); i += 64)
            store16(a.out + row * HO + (int64_t)h0 * C::DV + 8 * i, u32x4{0, 0, 0, 0});
        }
        continue;
      }
      k_lo = r.lo;
      k_hi = r.nsplit > 0 ? min(r.hi, k_lo + a.split_tokens) : k_lo;
    }

    // Q as the B operand: lane (q, l16) holds head l16, channels 32 ks + 8 q + [0, 8),
    // rotated on its suffix window
    const bool head_ok = l16 < a.chunk_heads;
    h8 qf[C::KS];
    {
      const uint16_t* qrow = a.query + (int64_t)r.t * HQ + (int64_t)(h0 + l16) * C::D;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        u32x4 v = u32x4{0, 0, 0, 0};
        const int c = 4 * ks + q;
        if (head_ok) {
          v = load16(qrow + 8 * c);
          // the rotary window lies past the V channels (checked on the host)
          if (ks >= C::DV / 32 && chunk_rotated(c, a.rotary_offset, a.rotary_dim)) {
            const int off = a.rotary_offset;
            float rr[8];
            rotate_chunk(qrow + off, v, c - off / 8, r.pos, a.cos, a.sin, a.rotary_dim,
                         a.rotary_interleaved, a.rotary_rows, rr);
            v = pack8(rr);
          }
        }
        qf[ks] = as_h8(v);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    f4 acc[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    const int32_t* bt = sl.block_table + (int64_t)r.b * sl.maxblk;

    for (int seg_lo = k_lo; seg_lo < k_hi;) {
      const int first_bi = seg_lo >> shift;
      const int seg_hi = min(k_hi, (first_bi + C::TBL) << shift);
      const int n_bi = ((seg_hi - 1) >> shift) - first_bi + 1;
      bool hole = false;
      for (int i = lane; i < n_bi; i += 64) {
        const int bi = first_bi + i;
        int v = bi < sl.maxblk ? bt[bi] : -1;
        if (v >= sl.num_blocks) v = -1;
        hole |= v < 0;
        tbl[i] = v;
      }
      const bool any_hole = __any(hole);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      const int ntile = (seg_hi - seg_lo + C::KT - 1) / C::KT;
      // Tile `t`'s rows into registers (main parts: one 1 KB load per row;
      // rotary tails: one per 8 rows), then into this wave's LDS tile: the
      // next tile's loads stay in flight while this one is computed.
      u32x4 stg[C::KT + C::KT / 8];
      auto stage_load = [&](int t) {
        const int k0 = seg_lo + t * C::KT;
        const uint32_t mine = mla_row_offset(tbl, first_bi, shift, k0 + (lane & (C::KT - 1)), seg_hi);
#pragma unroll
        for (int r = 0; r < C::KT; ++r) {
          const uint32_t base = __builtin_amdgcn_readlane(mine, r);
          stg[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(srd, base + 16 * lane, 0, 0));
        }
        const int rr = lane >> 3, cc = (lane & 7) ^ (rr & 7);
#pragma unroll
        for (int g = 0; g < C::KT / 8; ++g) {
          const uint32_t base = (uint32_t)__shfl((int)mine, 8 * g + rr, 64);
          stg[C::KT + g] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(srd, base + 2 * (C::DV + 8 * cc), 0, 0));
        }
      };
      auto stage_store = [&](char* buf) {
#pragma unroll
        for (int r = 0; r < C::KT; ++r)
          *reinterpret_cast<u32x4*>(buf + r * C::MAIN + 16 * lane) = stg[r];
#pragma unroll
        for (int g = 0; g < C::KT / 8; ++g)
          *reinterpret_cast<u32x4*>(buf + C::KT * C::MAIN + 8 * g * C::TAIL + 16 * lane) =
              stg[C::KT + g];
      };
      stage_load(0);
      for (int it = 0; it < ntile; ++it) {
        const int k0 = seg_lo + it * C::KT;
        const bool more = it + 1 < ntile;
        char* tile = s_k[wave];
        const uint16_t* kmain = reinterpret_cast<const uint16_t*>(tile);
        const uint16_t* ktail = reinterpret_cast<const uint16_t*>(tile + C::KT * C::MAIN);
        stage_store(tile);                    // (waits for this tile's loads)
        if (more) stage_load(it + 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- S^T = K . Q^T: two 16-key blocks over the 576 channels ----
        // operand reads run kAheadK products ahead of their MFMAs (the two
        // 16-key blocks alternate, so consecutive products are independent)
        f4 s[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
        auto kread = [&](int i) __attribute__((always_inline)) {
          const int sb = i & 1, ks = i >> 1;
          const int rk = 16 * sb + l16;
          const uint16_t* src =
              ks < C::DV / 32 ? kmain + rk * (C::MAIN / 2) + 32 * ks + 8 * q
                              : ktail + 8 * tail_slot(rk, 4 * (ks - C::DV / 32) + q);
          return *reinterpret_cast<const h8*>(src);
        };
        {
          constexpr int NQ = 2 * C::KS;
          h8 kf[kAheadK];
#pragma unroll
          for (int i = 0; i < kAheadK; ++i) kf[i] = kread(i);
#pragma unroll
          for (int i = 0; i < NQ; ++i) {
            s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[i % kAheadK], qf[i >> 1],
                                                              s[i & 1], 0, 0, 0);
            if (i + kAheadK < NQ) kf[i % kAheadK] = kread(i + kAheadK);
            __builtin_amdgcn_sched_barrier(0);
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
              v = tanh_fast(v * a.cap_in) * a.cap_out;
            else
              v = v * a.score_scale;
            if (edge) {
              const int key = k0 + 16 * sb + 4 * q + rr;
              const bool ok = key < seg_hi && tbl[(key >> shift) - first_bi] >= 0;
              v = ok ? v : kNegInf;
            }
            x[4 * sb + rr] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = lane_max32(lane_max16(mx));
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

        // ---- O^T += V^T . P^T, V^T read from the K tile (channels < 512) ----
        auto vread = [&](int db) __attribute__((always_inline)) {
          v4s part[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
            part[sb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(
                    kmain + (16 * sb + 4 * q + (l16 >> 2)) * (C::MAIN / 2) + 16 * db +
                    4 * (l16 & 3)));
          h8 va;
          __builtin_memcpy(&va, part, 16);
          return va;
        };
        {
          h8 vf[kAheadV];
#pragma unroll
          for (int i = 0; i < kAheadV; ++i) vf[i] = vread(i);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[db % kAheadV], pf, acc[db], 0, 0, 0);
            if (db + kAheadV < C::DB) vf[db % kAheadV] = vread(db + kAheadV);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // every read of the tile has returned (the products above consumed
        // them): the next tile's stores may overwrite it
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      seg_lo = seg_hi;
      __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: lane (q, l16) holds head l16, channels 16 db + 4 q + [0, 4) ----
    const float lt = lane_sum32(lane_sum16(lsum));
    if (head_ok) {
      const int h = h0 + l16;
      if (r.nsplit <= 1) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        uint16_t* orow = a.out + (int64_t)r.t * HO + (int64_t)h * C::DV;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          uint2 w;
          w.x = (uint32_t)f2h(acc[db][0] * inv) | ((uint32_t)f2h(acc[db][1] * inv) << 16);
          w.y = (uint32_t)f2h(acc[db][2] * inv) | ((uint32_t)f2h(acc[db][3] * inv) << 16);
          *reinterpret_cast<uint2*>(orow + 16 * db + 4 * q) = w;
        }
      } else {
        const int64_t pidx = ((int64_t)row * a.num_heads + h) * a.max_splits + split;
        float* po = a.part_o + pidx * C::DV;
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

// Shared mode for many heads, in wave pairs: a workgroup of 8 waves takes
// four head chunks (64 heads) of one (row, split); the two waves of a pair
// share a head chunk and split its work -- the QK product over the channel
// halves (k-steps 0..8 and 9..17, whose partial scores are summed through LDS),
// the PV product over the output channel halves (0..255 and 256..511).  A
// wave then holds half the Q fragments and half the accumulator, so two
// waves fit each SIMD and one's softmax and barriers run under the other's
// products.  Waves 0..3 copy the tiles into the double buffer as in the
// four-wave shared mode.
template <bool SOFTCAP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void mla_pair_kernel(const DecodeArgs a) {
  using C = MlaCfg;
  constexpr int KH = C::KS / 2;        // 9 k-steps per half
  constexpr int DBH = C::DB / 2;       // 16 output blocks per half
  __shared__ __attribute__((aligned(16))) char s_k[2][C::TILE];
  __shared__ __attribute__((aligned(16))) f4 s_sx[C::WAVES][2][2][64];   // [pair][half][block][lane]
  __shared__ int32_t s_tbl[C::TBL];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..7
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const SeqLayout& sl = a.s;
  const int HC = a.head_chunks;
  const int64_t HQ = (int64_t)a.num_heads * C::D;
  const int64_t HO = (int64_t)a.num_heads * C::DV;
  const int HG = (HC + C::WAVES - 1) / C::WAVES;   // items per entry: groups of 4 chunks
  const int total = a.listed ? (*a.entry_count) * HG : a.rows * HG;
  int32_t* tbl = s_tbl;
  const int shift = sl.block_shift;
  const bool copier = wave < C::WAVES;   // waves 0..3 copy a quarter of every tile each
  const int64_t pool_bytes = (sl.num_blocks << shift) * (int64_t)(2 * C::D);
  const __amdgpu_buffer_rsrc_t srd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.key_cache, (short)0, (int)(uint32_t)min(pool_bytes, (int64_t)0xFFFFFFFF),
      0x00020000);

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int e = item / HG;
    const int hc = (item - e * HG) * C::WAVES + pair;
    const bool chunk_ok = hc < HC;   // a pair past the last chunk only helps copy
    const int h0 = hc * a.chunk_heads;

    int row, split, k_lo, k_hi;
    RowInfo r;
    if (a.listed) {
      const DecodeEntry en = a.entries[e];
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
      if (!resolve_row(sl, 1, row, a.window, a.split_tokens, a.max_splits, r, orphan)) {
        if (orphan && row < sl.tokens && chunk_ok) {   // token owned by no request: zero
          for (int i = lane; i < a.chunk_heads * (C::DV / 16); i += 64) {
            const int hh = i / (C::DV / 16), cc = i % (C::DV / 16);
            store16(a.out + row * HO + (int64_t)(h0 + hh) * C::DV + half * (C::DV / 2) + 8 * cc,
                    u32x4{0, 0, 0, 0});
          }
        }
        continue;
      }
      k_lo = r.lo;
      k_hi = r.nsplit > 0 ? min(r.hi, k_lo + a.split_tokens) : k_lo;
    }

    // this wave's half of Q as the B operand: lane (q, l16) holds head l16,
    // channels 32 (KH half + j) + 8 q + [0, 8), rotated on its suffix window
    const bool head_ok = chunk_ok && l16 < a.chunk_heads;
    h8 qf[KH];
    {
      const uint16_t* qrow = a.query + (int64_t)r.t * HQ + (int64_t)(h0 + l16) * C::D;
#pragma unroll
      for (int j = 0; j < KH; ++j) {
        const int ks = KH * half + j;
        u32x4 v = u32x4{0, 0, 0, 0};
        const int c = 4 * ks + q;
        if (head_ok) {
          v = load16(qrow + 8 * c);
          // the rotary window lies past the V channels (checked on the host)
          if (ks >= C::DV / 32 && chunk_rotated(c, a.rotary_offset, a.rotary_dim)) {
            const int off = a.rotary_offset;
            float rr[8];
            rotate_chunk(qrow + off, v, c - off / 8, r.pos, a.cos, a.sin, a.rotary_dim,
                         a.rotary_interleaved, a.rotary_rows, rr);
            v = pack8(rr);
          }
        }
        qf[j] = as_h8(v);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    f4 acc[DBH];
#pragma unroll
    for (int i = 0; i < DBH; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    const int32_t* bt = sl.block_table + (int64_t)r.b * sl.maxblk;

    for (int seg_lo = k_lo; seg_lo < k_hi;) {
      const int first_bi = seg_lo >> shift;
      const int seg_hi = min(k_hi, (first_bi + C::TBL) << shift);
      const int n_bi = ((seg_hi - 1) >> shift) - first_bi + 1;
      bool hole = false;
      for (int i = threadIdx.x; i < n_bi; i += 64 * 2 * C::WAVES) {
        const int bi = first_bi + i;
        int v = bi < sl.maxblk ? bt[bi] : -1;
        if (v >= sl.num_blocks) v = -1;
        hole |= v < 0;
        tbl[i] = v;
      }
      const bool any_hole = __syncthreads_or(hole);

      const int ntile = (seg_hi - seg_lo + C::KT - 1) / C::KT;
      auto copy = [&](int t, char* buf) {
        if (copier)
          mla_copy_rows<1>(srd, buf, tbl, first_bi, shift, seg_lo + t * C::KT, seg_hi, lane, wave);
      };
      copy(0, s_k[0]);
      if (ntile > 1) copy(1, s_k[1]);
      for (int it = 0; it < ntile; ++it) {
        const int k0 = seg_lo + it * C::KT;
        const bool more = it + 1 < ntile;
        char* tile = s_k[it & 1];
        const uint16_t* kmain = reinterpret_cast<const uint16_t*>(tile);
        const uint16_t* ktail = reinterpret_cast<const uint16_t*>(tile + C::KT * C::MAIN);
        // this wave's part of tile it has landed (tile it + 1's may be in
        // flight: 9 instructions), then everyone's
        if (more)
          __builtin_amdgcn_s_waitcnt(0x0F79);   // vmcnt(9)
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();

        // ---- this wave's half of S^T = K . Q^T (k-steps KH half ..) ----
        f4 s[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
        if (chunk_ok) {
          auto kread = [&](int i) __attribute__((always_inline)) {
            const int sb = i & 1, ks = KH * half + (i >> 1);
            const int rk = 16 * sb + l16;
            const uint16_t* src =
                ks < C::DV / 32 ? kmain + rk * (C::MAIN / 2) + 32 * ks + 8 * q
                                : ktail + 8 * tail_slot(rk, 4 * (ks - C::DV / 32) + q);
            return *reinterpret_cast<const h8*>(src);
          };
          constexpr int NQ = 2 * KH;
          h8 kf[kAheadK];
#pragma unroll
          for (int i = 0; i < kAheadK; ++i) kf[i] = kread(i);
#pragma unroll
          for (int i = 0; i < NQ; ++i) {
            s[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[i % kAheadK], qf[i >> 1],
                                                              s[i & 1], 0, 0, 0);
            if (i + kAheadK < NQ) kf[i % kAheadK] = kread(i + kAheadK);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- the pair's partial scores summed through LDS (both waves form
        // the same sum: fp32 addition commutes) ----
        s_sx[pair][half][0][lane] = s[0];
        s_sx[pair][half][1][lane] = s[1];
        __syncthreads();
        {
          const f4 o0 = s_sx[pair][1 - half][0][lane], o1 = s_sx[pair][1 - half][1][lane];
          s[0] = half == 0 ? s[0] + o0 : o0 + s[0];
          s[1] = half == 0 ? s[1] + o1 : o1 + s[1];
        }
        if (chunk_ok) {
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
                v = tanh_fast(v * a.cap_in) * a.cap_out;
              else
                v = v * a.score_scale;
              if (edge) {
                const int key = k0 + 16 * sb + 4 * q + rr;
                const bool ok = key < seg_hi && tbl[(key >> shift) - first_bi] >= 0;
                v = ok ? v : kNegInf;
              }
              x[4 * sb + rr] = v;
              mx = fmaxf(mx, v);
            }
          }
          mx = lane_max32(lane_max16(mx));
          if (__any(mx > m + kRescaleSlack)) {
            const float mn = mx > m + kRescaleSlack ? mx : m;
            const float alpha = exp2_fast(m - (mn == kNegInf ? 0.f : mn));
            m = mn;
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < DBH; ++i) acc[i] *= alpha;
          }
          const float mu = m == kNegInf ? 0.f : m;
          h8 pf;   // keys 4q + (0..3) of both 16-key blocks, in that order
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = exp2_fast(x[i] - mu);
            lsum += p;
            pf[i] = (_Float16)p;
          }

          // ---- this wave's half of O^T += V^T . P^T (channels 256 half ..) ----
          auto vread = [&](int db) __attribute__((always_inline)) {
            v4s part[2];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
              part[sb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4s*)(
                      kmain + (16 * sb + 4 * q + (l16 >> 2)) * (C::MAIN / 2) +
                      16 * (DBH * half + db) + 4 * (l16 & 3)));
            h8 va;
            __builtin_memcpy(&va, part, 16);
            return va;
          };
          h8 vf[kAheadV];
#pragma unroll
          for (int i = 0; i < kAheadV; ++i) vf[i] = vread(i);
#pragma unroll
          for (int db = 0; db < DBH; ++db) {
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[db % kAheadV], pf, acc[db], 0, 0, 0);
            if (db + kAheadV < DBH) vf[db % kAheadV] = vread(db + kAheadV);
            __builtin_amdgcn_sched_barrier(0);
          }
        }   // chunk_ok
        // every read of the tile (and of the score exchange) has returned: a
        // later tile's copy may overwrite the tile, the next scores the slots
        __syncthreads();
        if (it + 2 < ntile) copy(it + 2, tile);
      }
      seg_lo = seg_hi;
      __syncthreads();   // the table is restaged for the next segment
    }

    // ---- epilogue: lane (q, l16) holds head l16, channels 256 half + 16 db + 4 q + [0, 4) ----
    const float lt = lane_sum32(lane_sum16(lsum));
    if (head_ok) {
      const int h = h0 + l16;
      const int cb = (C::DV / 2) * half;
      if (r.nsplit <= 1) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        uint16_t* orow = a.out + (int64_t)r.t * HO + (int64_t)h * C::DV + cb;
#pragma unroll
        for (int db = 0; db < DBH; ++db) {
          uint2 w;
          w.x = (uint32_t)f2h(acc[db][0] * inv) | ((uint32_t)f2h(acc[db][1] * inv) << 16);
          w.y = (uint32_t)f2h(acc[db][2] * inv) | ((uint32_t)f2h(acc[db][3] * inv) << 16);
          *reinterpret_cast<uint2*>(orow + 16 * db + 4 * q) = w;
        }
      } else {
        const int64_t pidx = ((int64_t)row * a.num_heads + h) * a.max_splits + split;
        float* po = a.part_o + pidx * C::DV + cb;
#pragma unroll
        for (int db = 0; db < DBH; ++db) *reinterpret_cast<f4*>(po + 16 * db + 4 * q) = acc[db];
        if (q == 0 && half == 0) {
          a.part_ml[2 * pidx] = m;
          a.part_ml[2 * pidx + 1] = lt;
        }
      }
    }
  }
}

template <bool SOFTCAP>
int mla_occupancy() {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mla_kernel<SOFTCAP>, 256, 0) !=
            hipSuccess ||
        n <= 0)
      n = 1;
    cached = n;
  }
  return cached;
}

}  // namespace

int mla_workgroups_per_cu(bool softcap) {
  return softcap ? mla_occupancy<true>() : mla_occupancy<false>();
}

hipError_t launch_mla(const DecodeArgs& a, int workgroups, hipStream_t st) {
  const dim3 grid(workgroups), block(64 * MlaCfg::WAVES);
  // shared mode once a workgroup's four waves each have a head chunk
  const bool shared = a.head_chunks >= MlaCfg::WAVES;
  if (shared) {
    const dim3 pair_block(2 * 64 * MlaCfg::WAVES);
    if (a.use_softcap)
      launch_kernel(mla_pair_kernel<true>, grid, pair_block, st, a);
    else
      launch_kernel(mla_pair_kernel<false>, grid, pair_block, st, a);
  } else {
    if (a.use_softcap)
      launch_kernel(mla_kernel<true>, grid, block, st, a);
    else
      launch_kernel(mla_kernel<false>, grid, block, st, a);
  }
  return hipGetLastError();
}

}  // namespace pa
