// Prefill / chunked-prefill attention, 8-wave kernel for the wide head
// (D = 256): 16 query rows per wave, so that a wave's registers (output
// accumulator, query fragments, two score tiles, the staged loads of the next
// tiles) fit in half of a SIMD's register file and two waves share every
// SIMD: while one wave computes its softmax or waits on LDS, the other keeps
// the matrix core busy.
//
// It computes what the 4-wave kernel in prefill.hip computes: online-softmax
// tiled attention (GroupQueryAttention CPU Implementation Notes, "Flash
// Attention Path") with softcap applied to the scaled score before masking
// (PagedAttention -- CUDA Design Document, section 8.5 note), causal masking
// and the window of W positions ending at the query (section 4.5), keys
// addressed one row at a time through the block table.
//
// One workgroup = 8 waves = 128 query rows (token x head-in-group, token
// major) of one kv head; every K/V tile in LDS is shared by the 8 waves.
// Each wave owns 16 rows and computes
//   S^T[key][row] = K[key][:] . Q[row][:]          (v_mfma_f32_16x16x32_f16)
// whose accumulator (lane l: keys 16 kb + 4 (l / 16) + 0..3 of row l % 16) is
// the B operand of
//   O^T[d][row] += V^T[d][key] . P^T[key][row]     (v_mfma_f32_16x16x32_f16)
// once the keys of each 32-key k-step are taken in "slot order":
//   slot 8 q + i     <-> key 4 q + i        (i < 4)
//   slot 8 q + 4 + i <-> key 16 + 4 q + i
// K tiles of 64 keys move from the pool straight into LDS (buffer loads with
// an LDS destination, 1 KB per instruction: the buffer form, unlike the
// global one, leaves the compiler free to wait on individual LDS reads).
// V tiles are loaded into registers one step ahead and written to LDS
// transposed (V^T rows of 64 keys in slot order), the 8 x 8 blocks
// transposed in registers with lane swaps and byte permutes.  Both MFMA
// operands are then plain 16-byte LDS reads.  The 16-byte slot groups of
// V^T row d sit at group ^ ((d / 16) % 8): the rows written together are 8
// apart and would otherwise share their banks.  Byte offsets into the pool
// are 32-bit: the pool of one cache is smaller than 4 GiB (checked by the
// host); keys that must read as zero use an offset past the buffer's end.
// The tile pipeline: K one tile ahead of V, double-buffered LDS tiles, the
// QK product of the next tile interleaved with the softmax of the current
// one, one barrier per tile, scores in log2 units with a lazily raised
// running max.
//
// Quantized pools (PagedAttention -- CUDA Design Document, section 8.5,
// phase 3): K rows load as byte codes into registers where the fp16 kernel
// issues its direct loads, and are written into the same LDS slots as fp16
// values (every int8 and e4m3fn value is an fp16 value) just before the
// step's barrier; V codes load into registers one step ahead like fp16 V and
// become fp16 right before their transpose.  A per-tensor K scale joins the
// score scale, a per-channel one multiplies Q; the V scale multiplies the
// output accumulator.
#include <type_traits>

#include "prefill_common.h"

namespace pa {

namespace {

template <int D>
struct Rows16Cfg {
  static_assert(D == 256, "the 8-wave kernel is laid out for 256-channel heads");
  static constexpr int WAVES = 8;
  static constexpr int KT = 64;              // keys per tile
  static constexpr int KS = D / 32;          // QK k-steps over the head dim (32 channels)
  static constexpr int DB = D / 16;          // 16-channel output blocks
  static constexpr int CH = D / 8;           // 16-byte chunks per key row
  static constexpr int RPS = 64 / CH;        // key rows per 1 KB slot (one direct load)
  static constexpr int NS = 32 / RPS;        // slots per 32-key block
  static constexpr int SLOTS = KT / RPS;     // K slots per tile
  static constexpr int DMA = SLOTS / WAVES;  // direct K loads per wave per tile
  static constexpr int KSLOT = 1024 + 32;    // K slot stride in LDS (bytes)
  static constexpr int VROW = 2 * KT + 32;   // V^T row stride in LDS (bytes); both strides
                                             // are the fastest measured for the reads
  static constexpr int SEGT = 512;           // block-table entries staged per segment
  static constexpr int PIPE = 1;             // k-steps of K operands read ahead
  static constexpr int VPIPE = 2;            // V operands read ahead
};

__device__ __forceinline__ void lane_swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void lane_swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Transpose 8 x 8 fp16 blocks held by lanes m, m + 16, m + 32, m + 48:
// before, the lane of group G holds rows 2G (c0) and 2G + 1 (c1) of its block
// (8 columns each); after, it holds columns 2G (c0) and 2G + 1 (c1) (8 rows
// each).  The lane-group bits are exchanged with the dword bits by two lane
// swaps, the chunk bit with the half-word bit by byte permutes.
__device__ __forceinline__ void transpose8x8(u32x4& c0, u32x4& c1) {
  uint32_t x0[4] = {c0[0], c0[1], c0[2], c0[3]};
  uint32_t x1[4] = {c1[0], c1[1], c1[2], c1[3]};
  lane_swap32(x0[0], x0[2]);
  lane_swap32(x0[1], x0[3]);
  lane_swap32(x1[0], x1[2]);
  lane_swap32(x1[1], x1[3]);
  lane_swap16(x0[0], x0[1]);
  lane_swap16(x0[2], x0[3]);
  lane_swap16(x1[0], x1[1]);
  lane_swap16(x1[2], x1[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    c0[w] = __builtin_amdgcn_perm(x1[w], x0[w], 0x05040100u);   // low halves
    c1[w] = __builtin_amdgcn_perm(x1[w], x0[w], 0x07060302u);   // high halves
  }
}

// CT: element type of the pools (kCacheF16, or int8 / e4m3fn codes).
template <int D, bool SOFTCAP, int CT>
__global__ __launch_bounds__(512) void prefill16_kernel(const PrefillArgs a) {
  using C = Rows16Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char K0[C::SLOTS * C::KSLOT];
  __shared__ __attribute__((aligned(1024))) char K1[C::SLOTS * C::KSLOT];
  __shared__ __attribute__((aligned(1024))) char V0[D * C::VROW];
  __shared__ __attribute__((aligned(1024))) char V1[D * C::VROW];
  __shared__ int32_t s_tbl[C::SEGT];
  __shared__ int sh_b, sh_tile, sh_tb, sh_ql, sh_past;

  const SeqLayout& sl = a.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  __builtin_assume(wave >= 0 && wave < C::WAVES);
  const int l16 = lane & 15;   // the lane's row within the wave (MFMA layouts)
  const int q4 = lane >> 4;    // the lane's 16-lane group
  const LogicalBlock lb = logical_block();   // XCD-aware order
  const int kvh = lb.y;
  const int g = a.group;
  const int64_t HD = (int64_t)a.num_heads * D;

  if (lb.x == a.tiles * a.chunks) {
    // tokens owned by no request get zero rows (this kv head's columns)
    const int t0 = max(sl.cum[sl.batch], 0);
    const int width = g * (D / 8);
    for (int64_t i = tid; i < (int64_t)(sl.tokens - min(t0, sl.tokens)) * width; i += 512) {
      const int t = t0 + (int)(i / width);
      const int cc = (int)(i % width);
      store16(a.out + t * HD + (int64_t)kvh * g * D + 8 * cc, u32x4{0, 0, 0, 0});
    }
    return;
  }

  if (wave == 0) {
    int fb, ft, tb, ql, ps;
    find_tile(sl, g, lb.x / a.chunks, lane, fb, ft, tb, ql, ps);
    if (lane == 0) {
      sh_b = fb;
      sh_tile = ft;
      sh_tb = tb;
      sh_ql = ql;
      sh_past = ps;
    }
  }
  __syncthreads();
  const int b = __builtin_amdgcn_readfirstlane(sh_b);
  if (b < 0) return;
  const int tile = __builtin_amdgcn_readfirstlane(sh_tile);

  const int t_begin = __builtin_amdgcn_readfirstlane(sh_tb);
  const int q_len = __builtin_amdgcn_readfirstlane(sh_ql);
  const int past = __builtin_amdgcn_readfirstlane(sh_past);
  const int cap = sl.maxblk << sl.block_shift;
  const int shift = sl.block_shift;
  const int bmask = (1 << shift) - 1;
  const int32_t* bt = sl.block_table + (int64_t)b * sl.maxblk;
  const uint32_t tok_stride32 = (uint32_t)(a.kv_heads * D);   // Hkv * D < 2^24
  const uint16_t* kbase = a.key_cache + (int64_t)kvh * D;
  const uint16_t* vbase = a.value_cache + (int64_t)kvh * D;
  // buffer over this kv head's part of the key pool (bytes from kbase on)
  const int64_t kbytes = ((sl.num_blocks << shift) * a.kv_heads * D - (int64_t)kvh * D) * 2;
  const __amdgpu_buffer_rsrc_t ksrd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kbase, (short)0, (int)(uint32_t)min(kbytes, (int64_t)0xFFFFFFFF), 0x00020000);
  // quantized pools: byte arrays of codes, one byte per element
  constexpr bool kCodes = CT != kCacheF16;
  const char* kcode = reinterpret_cast<const char*>(a.key_cache) + (int64_t)kvh * D;
  const char* vcode = reinterpret_cast<const char*>(a.value_cache) + (int64_t)kvh * D;
  // a per-tensor K scale joins the score scale (and the softcap's input
  // scale); a per-channel one is folded into Q below
  float score_scale = a.score_scale, cap_in2 = a.cap_in2;
  bool k_per_channel = false;
  if constexpr (kCodes) {
    if (a.k_quant == kQuantChannel) {
      k_per_channel = true;
    } else {
      const float ks = a.k_scale[0];
      score_scale *= ks;
      cap_in2 *= ks;
    }
  }

  // this lane's query row
  const int R = tile * kPrefillRows + wave * 16 + l16;
  const int j = R / g;
  const int hh = R - j * g;
  const bool row_ok = j < q_len && t_begin + j < sl.tokens;
  const int pos = row_ok ? past + j : -1;
  const int t = t_begin + j;
  const int head = kvh * g + hh;

  const TileKeys tk = tile_keys(tile, q_len, past, g, a.window, cap, a.chunks, a.piece_tiles);
  const int piece = lb.x - (lb.x / a.chunks) * a.chunks;
  const int pieces = tk.pieces;
  if (piece >= pieces) return;
  const int hi = tk.hi;
  const int lo = tk.lo;
  const int wj0 = min((tile * kPrefillRows + wave * 16) / g, q_len - 1);
  const int wj1 = min((tile * kPrefillRows + wave * 16 + 15) / g, q_len - 1);
  const int wpos_min = past + wj0;
  const int wpos_max = past + wj1;

  // Q fragments (B operand): row l16, channels 32 ks + 8 q4 .. +7
  // all chunk loads first (one memory round trip), then the chunks that
  // RoPE rotates or a per-channel K scale multiplies
  h8 qf[C::KS];
  const uint16_t* qrow = a.query + (int64_t)t * HD + (int64_t)head * D;
  if (row_ok) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(load16(qrow + 8 * (4 * ks + q4)));
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(u32x4{0, 0, 0, 0});
  }
  if (row_ok && (a.rotary_dim > 0 || k_per_channel)) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int c = 4 * ks + q4;
      const bool rot = chunk_rotated(c, a.rotary_offset, a.rotary_dim);
      if (rot || k_per_channel) {
        const int off = rot ? a.rotary_offset : 0;
        u32x4 v;
        __builtin_memcpy(&v, &qf[ks], 16);
        float rr[8];
        rotate_chunk(qrow + off, v, c - off / 8, pos, a.cos, a.sin, rot ? a.rotary_dim : 0,
                     a.rotary_interleaved, a.rotary_rows, rr);
        if (k_per_channel) {
          float ks8[8];
          channel_scales(a.k_scale, kQuantChannel, kvh, D, 8 * c, ks8);
#pragma unroll
          for (int e = 0; e < 8; ++e) rr[e] *= ks8[e];
        }
        qf[ks] = as_h8(pack8(rr));
      }
    }
  }

  f4 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  const int kt_begin = tk.all_begin + piece * tk.per_piece * C::KT;
  const int ntiles = min(tk.per_piece, tk.all_tiles - piece * tk.per_piece);
  int seg_first = -1;
  bool wg_hole = false;

  auto stage_table = [&](int k) {
    __syncthreads();
    seg_first = k >> shift;
    const int last_bi = (hi - 1) >> shift;
    bool hole = false;
    for (int i = tid; i < C::SEGT; i += 64 * C::WAVES) {
      const int bi = seg_first + i;
      int v = -1;
      if (bi <= last_bi && bi < sl.maxblk) {
        v = bt[bi];
        if (v >= sl.num_blocks) v = -1;
        const int k0 = bi << shift;
        if (v < 0 && k0 + bmask >= lo && k0 < hi) hole = true;
      }
      s_tbl[i] = v;
    }
    wg_hole = __syncthreads_or(hole) || wg_hole;
  };

  auto kbuf = [&](auto B) -> char* { if constexpr (B() == 0) return K0; else return K1; };
  auto vbuf = [&](auto B) -> char* { if constexpr (B() == 0) return V0; else return V1; };
  auto kt_of = [&](int tt) { return kt_begin + tt * C::KT; };

  // ---- K tile loads: wave w fills slots w, w + 8, ...; lane i of a slot
  // load moves chunk i % CH of key row i / CH of the slot.  Key row r (0..63)
  // of a tile lives in slot (r / 32) NS + r % NS at row position (r % 32) / NS.
  auto row_k = [&](int tt, int mi) -> uint32_t {
    const int slot = wave + C::WAVES * mi;
    const int tau = kt_of(tt) + (slot / C::NS) * 32 + (slot % C::NS) + C::NS * (lane / C::CH);
    const bool in = (tt < ntiles) & (tau >= lo) & (tau < hi);
    const int v = s_tbl[in ? (tau >> shift) - seg_first : 0] | (in ? 0 : -1);
    return v < 0 ? ~0u : ((uint32_t)v << shift) | (uint32_t)(tau & bmask);
  };
  // quantized pools: the lane's eight codes of a K row (a zero row reads the
  // zero block: code 0 is +0), and their fp16 values written into the lane's
  // 16 bytes of the slot the direct load would fill
  auto load_kcode = [&](uint32_t row) -> u32x2 {
    const int64_t off = row != ~0u ? (int64_t)row * tok_stride32 + 8 * (lane % C::CH)
                                   : reinterpret_cast<const char*>(g_zero_row) - kcode;
    return *reinterpret_cast<const u32x2*>(kcode + off);
  };
  auto put_k = [&](u32x2 c, char* kb, int mi) {
    *reinterpret_cast<u32x4*>(kb + (wave + C::WAVES * mi) * C::KSLOT + 16 * lane) =
        codes_to_f16<CT>(c);
  };
  auto dma_k = [&](uint32_t row, char* kb, int mi) {
    const uint32_t off = row != ~0u ? (row * tok_stride32 + 8 * (lane % C::CH)) * 2 : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ksrd, (__attribute__((address_space(3))) void*)(kb + (wave + C::WAVES * mi) * C::KSLOT), 16,
        off, 0, 0, 0);
  };
  // ---- V tile loads: wave w moves key group w (slots 8w .. 8w + 7 of the
  // tile); the lane of group G = lane / 16 moves keys 2G + x (x = 0, 1) of
  // the group, channel chunks m + 16 y (m = lane % 16, y = 0, 1) ----
  const int lm = lane & 15;
  const int lg = lane >> 4;
  // tile-relative key of slot 8 wave + jj
  auto slot_key = [&](int jj) {
    return 32 * (wave >> 2) + (jj < 4 ? 4 * (wave & 3) + jj : 16 + 4 * (wave & 3) + jj - 4);
  };
  const int key0 = slot_key(2 * lg), key1 = slot_key(2 * lg + 1);
  // pool row of this lane's key x of tile tt, or ~0 when the key is outside
  // [lo, hi), in an unmapped block or past this workgroup's tiles (then a
  // zero row is loaded).  Pools hold fewer than 2^32 rows.
  auto row_v = [&](int tt, int x) -> uint32_t {
    const int tau = kt_of(tt) + (x ? key1 : key0);
    const bool in = (tt < ntiles) & (tau >= lo) & (tau < hi);
    const int v = s_tbl[in ? (tau >> shift) - seg_first : 0] | (in ? 0 : -1);
    return v < 0 ? ~0u : ((uint32_t)v << shift) | (uint32_t)(tau & bmask);
  };
  // element offset from `base` of chunk y of pool row `row` (a zero row for ~0)
  auto chunk_off = [&](uint32_t row, const uint16_t* base, int y) -> int64_t {
    const int ch = 8 * (lm + 16 * y);
    return row != ~0u ? (int64_t)((uint64_t)row * tok_stride32 + ch) : (g_zero_row + ch) - base;
  };
  // staged loads: [x][y] = chunk y of key x (codes: in vcodes until widened)
  u32x4 vreg[2][2];
  u32x2 vcodes[2][2];
  auto load_v = [&](const uint32_t (&rows)[2]) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        if constexpr (kCodes) {
          const int ch = 8 * (lm + 16 * y);
          const int64_t off = rows[x] != ~0u
                                  ? (int64_t)((uint64_t)rows[x] * tok_stride32 + ch)
                                  : reinterpret_cast<const char*>(g_zero_row) - vcode;
          vcodes[x][y] = *reinterpret_cast<const u32x2*>(vcode + off);
        } else {
          vreg[x][y] = load16(vbase + chunk_off(rows[x], vbase, y));
        }
      }
  };
  // codes of chunk y of both keys as fp16 values, ready for the transpose
  auto widen_v = [&](int y) {
    if constexpr (kCodes) {
      vreg[0][y] = codes_to_f16<CT>(vcodes[0][y]);
      vreg[1][y] = codes_to_f16<CT>(vcodes[1][y]);
    }
  };
  // V^T transposed: after the transpose the lane holds channels 2G + x of
  // chunk m + 16 y for the group's 8 keys in slot order
  const int vw_group = 16 * (wave ^ ((lm >> 1) & 7));   // swizzled slot group of the writes
  auto write_v1 = [&](char* vb, int x, int y) {
    *reinterpret_cast<u32x4*>(vb + (8 * (lm + 16 * y) + 2 * lg + x) * C::VROW + vw_group) =
        vreg[x][y];
  };
  auto write_v = [&](char* vb) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      widen_v(y);
      transpose8x8(vreg[0][y], vreg[1][y]);
#pragma unroll
      for (int x = 0; x < 2; ++x) write_v1(vb, x, y);
    }
  };
  auto need_segment = [&](int tt) {
    const int last = min(kt_of(tt) + C::KT, hi) - 1;
    return (last >> shift) >= seg_first + C::SEGT;
  };

  // Per-lane parts of the operand addresses, opaque to the compiler so every
  // operand read is one base register plus an immediate.
  int koff = 16 * q4 + row_byte<D>(l16, C::KSLOT);
  int voff[4];   // V^T reads: lane group q4's slot group, swizzled by k = 0..3
#pragma unroll
  for (int k = 0; k < 4; ++k) voff[k] = l16 * C::VROW + 16 * (q4 ^ k);
  asm("" : "+v"(koff), "+v"(voff[0]), "+v"(voff[1]), "+v"(voff[2]), "+v"(voff[3]));
  // A operand of S^T = K Q^T: key 16 kb + l16, channels 32 ks + 8 q4 .. +7
  auto kread = [&](const char* kt, int ks, int kb) {
    return *reinterpret_cast<const h8*>(kt + row_byte<D>(16 * kb, C::KSLOT) + 64 * ks);
  };
  // A operand of O^T += V^T P^T (MFMA i: block db = i % DB, k-step i / DB):
  // channel 16 db + l16, slots 32 ks + 8 q4 .. +7, i.e. slot group 4 ks + q4
  // stored at (4 ks + q4) ^ (db % 8)
  constexpr int NV = 2 * C::DB;
  auto vread = [&](const char* vt, int i) {
    const int db = i % C::DB, ks = i / C::DB;
    return *reinterpret_cast<const h8*>(vt + voff[db & 3] + 16 * db * C::VROW +
                                        64 * (ks ^ ((db >> 2) & 1)));
  };

  auto logit = [&](float x) {
    if constexpr (SOFTCAP)
      return a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_fast(x * cap_in2) + 1.0f));
    else
      return x * score_scale;
  };
  // a row's tile maximum in log2 units; the row's four lanes agree
  auto tile_max = [&](const f4 (&s)[4]) {
    float mq[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mq[kb] = fmaxf(fmaxf(s[kb][0], s[kb][1]), fmaxf(s[kb][2], s[kb][3]));
    const float mx = xor32_max(xor16_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))));
    return mx == kNegInf ? kNegInf : logit(mx);
  };
  auto full_tile = [&](int kt0) {
    return kt0 >= lo && kt0 + C::KT <= hi && kt0 + C::KT - 1 <= wpos_min &&
           (a.window <= 0 || kt0 >= wpos_max - a.window + 1);
  };
  // accumulator entry i of block kb holds key kt0 + 16 kb + 4 q4 + i; keys
  // past the table's capacity (hi is then the capacity) are masked too
  auto pos_mask = [&](f4 (&s)[4], int kt0) {
    const int wlo = a.window > 0 ? pos - a.window + 1 : INT32_MIN;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = kt0 + 16 * kb + 4 * q4 + i;
        s[kb][i] = ((tau <= pos) & (tau >= wlo) & (tau < hi)) ? s[kb][i] : kNegInf;
      }
  };
  // keys outside [lo, hi) or in an unmapped block (a run of four keys never
  // straddles a block)
  auto hole_mask = [&](f4 (&s)[4], int kt0) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int tau0 = kt0 + 16 * kb + 4 * q4;
      const int bi = (tau0 >> shift) - seg_first;
      const int v = bi >= 0 && bi < C::SEGT ? s_tbl[bi] : -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = tau0 + i;
        if (!(v >= 0 && tau >= lo && tau < hi)) s[kb][i] = kNegInf;
      }
    }
  };

  // Probabilities p = 2^(logit - mu) of scores f0 .. f0 + n - 1 (f = 4 kb + i)
  // into the fp16 B operand of the PV product: k-step kb / 2, slot
  // 8 q4 + 4 (kb % 2) + i.  Their sums accumulate in part.
  auto softmax_part = [&](const f4 (&s)[4], float mu, h8 (&pf)[2], float (&part)[4], int f0,
                          int n) {
#pragma unroll
    for (int f = f0; f < f0 + n; ++f) {
      const int kb = f >> 2, i = f & 3;
      const float x = s[kb][i];
      float e;
      if constexpr (SOFTCAP) {
        // cap * tanh(y) - mu = (cap - mu) - 2 cap / (2^t + 1), t = 2y log2(e);
        // a masked score (t = -inf) gets -inf through t * 2^-120
        const float tt = x * cap_in2;
        const float r = __builtin_amdgcn_rcpf(exp2_fast(tt) + 1.0f);
        e = __builtin_fmaf(tt, 0x1p-120f, __builtin_fmaf(r, -2.0f * a.cap_out, a.cap_out - mu));
      } else {
        e = __builtin_fmaf(x, score_scale, -mu);
      }
      const float p = exp2_fast(e);
      part[i] += p;
      pf[kb >> 1][4 * (kb & 1) + i] = (_Float16)p;
    }
  };

  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  f4 sA[4], sB[4];
  float mxA = kNegInf, mxB = kNegInf;
  if (ntiles > 0) {
    stage_table(max(kt_begin, lo));
#pragma unroll
    for (int mi = 0; mi < C::DMA; ++mi) {
      if constexpr (kCodes) {
        put_k(load_kcode(row_k(0, mi)), K0, mi);
        put_k(load_kcode(row_k(1, mi)), K1, mi);
      } else {
        dma_k(row_k(0, mi), K0, mi);
        dma_k(row_k(1, mi), K1, mi);
      }
    }
    const uint32_t r0[2] = {row_v(0, 0), row_v(0, 1)};
    load_v(r0);
    wait_vmem();
    write_v(V0);
    // in flight into the first step: V of tile 1
    const uint32_t r1[2] = {row_v(1, 0), row_v(1, 1)};
    load_v(r1);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sA[kb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sA[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kread(K0 + koff, ks, kb), qf[ks], sA[kb], 0, 0, 0);
    if (!full_tile(kt_of(0))) pos_mask(sA, kt_of(0));
    mxA = tile_max(sA);
    __syncthreads();   // K buffer 0 is written by the first step
  }

  // One step: softmax and PV of key tile `it` (scores s_cur, V in buffer B)
  // while tile it + 1's scores are computed (K in buffer 1 - B); K of tile
  // it + 2 streams into LDS, the staged V of tile it + 1 is written to LDS
  // and the loads of V of tile it + 2 are issued.
  auto step = [&](int it, auto B, f4 (&s_cur)[4], f4 (&s_next)[4], float& mx_cur,
                  float& mx_next) {
    using NB = std::integral_constant<int, 1 - B()>;
    if (wg_hole) {   // uniform and rare
      hole_mask(s_cur, kt_of(it));
      mx_cur = tile_max(s_cur);
    }
    {
      const float mn = mx_cur > m + kRescaleSlack ? mx_cur : m;
      const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
      m = mn;
      lsum *= alpha;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      }
    }
    const float mu = m == kNegInf ? 0.f : m;
    {
      const int tl = min(it + 2, ntiles - 1);
      if (tl > it && need_segment(tl)) stage_table(max(kt_of(it + 1), lo));
    }

    // ---- region A: QK of tile it + 1 with the first half of tile it's
    // softmax and the direct loads of tile it + 2's K (each one's table
    // lookup a k-step earlier); the V rows of tile it + 2 are looked up ----
    h8 pf[2];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t vrows[2];
    u32x2 kc[kCodes ? C::DMA : 1];   // quantized pools: this step's K codes, written at its end
    {
      for (int kb = 0; kb < 4; ++kb) s_next[kb] = f4{0.f, 0.f, 0.f, 0.f};
      const char* kt = kbuf(NB{}) + koff;
      h8 kf[C::PIPE][4];
#pragma unroll
      for (int p = 0; p < C::PIPE; ++p)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) kf[p][kb] = kread(kt, p, kb);
      uint32_t krow_next = row_k(it + 2, 0);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          s_next[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks % C::PIPE][kb], qf[ks], s_next[kb], 0, 0, 0);
          if (ks + C::PIPE < C::KS) kf[ks % C::PIPE][kb] = kread(kt, ks + C::PIPE, kb);
        }
        if (ks < C::DMA) {
          const uint32_t row = krow_next;
          if (ks + 1 < C::DMA) krow_next = row_k(it + 2, ks + 1);
          if constexpr (kCodes)
            kc[ks] = load_kcode(row);
          else
            dma_k(row, kbuf(B), ks);
        } else if (ks == C::DMA) {
          vrows[0] = row_v(it + 2, 0);
          vrows[1] = row_v(it + 2, 1);
        }
        softmax_part(s_cur, mu, pf, part, ks, 1);
        asm volatile("" ::"v"(part[0]), "v"(part[1]), "v"(part[2]), "v"(part[3]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- region B: PV of tile it with the second half of its softmax and
    // tile it + 1's row maximum; the staged V of tile it + 1 goes to LDS one
    // 16-byte write at a time, then the loads of V of tile it + 2 are
    // issued ----
    {
      const char* vt = vbuf(B);
      h8 vf[C::VPIPE];
#pragma unroll
      for (int p = 0; p < C::VPIPE; ++p) vf[p] = vread(vt, p);
      float mxr = kNegInf;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const int db = i % C::DB, ks = i / C::DB;
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[i % C::VPIPE], pf[ks], acc[db], 0, 0, 0);
        if (i + C::VPIPE < NV) vf[i % C::VPIPE] = vread(vt, i + C::VPIPE);
        // the V loads of the previous step have landed (this step's K
        // loads, issued after them, may still be in flight)
        if (i == 0) __builtin_amdgcn_s_waitcnt(0x0F70 | C::DMA);
        if (i == 17 || i == 21) {
          widen_v((i - 17) >> 2);
          transpose8x8(vreg[0][(i - 17) >> 2], vreg[1][(i - 17) >> 2]);
        } else if (i >= 18 && i <= 24 && (i & 1) == 0) {
          write_v1(vbuf(NB{}), (i >> 1) & 1, (i - 18) >> 2);
        } else if (i == 26) {
          load_v(vrows);
        }
        if (i < C::DB && (i & 1)) softmax_part(s_cur, mu, pf, part, 8 + (i >> 1), 1);
        if (i & 1) mxr = fmaxf(mxr, s_next[i >> 3][(i >> 1) & 3]);
        asm volatile("" ::"v"(mxr), "v"(part[0]), "v"(part[1]), "v"(part[2]), "v"(part[3]));
      }
      __builtin_amdgcn_sched_barrier(0);
      lsum += (part[0] + part[1]) + (part[2] + part[3]);
      mxr = xor32_max(xor16_max(mxr));
      mx_next = mxr == kNegInf ? kNegInf : logit(mxr);
    }
    if (it + 1 < ntiles && !full_tile(kt_of(it + 1))) {
      pos_mask(s_next, kt_of(it + 1));
      mx_next = tile_max(s_next);
    }
    if constexpr (kCodes) {
      // tile it + 2's K into buffer B, which no wave reads during this step
#pragma unroll
      for (int mi = 0; mi < C::DMA; ++mi) put_k(kc[mi], kbuf(B), mi);
    }
    // this step's K loads have landed (the V loads issued after them may
    // still be in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
    __syncthreads();
  };

  for (int it = 0; it < ntiles; it += 2) {
    step(it, Buf0{}, sA, sB, mxA, mxB);
    if (it + 1 < ntiles) step(it + 1, Buf1{}, sB, sA, mxB, mxA);
  }
  wait_vmem();   // loads past the last tile (zero rows) drain before the end

  const float lt = xor32_sum(xor16_sum(lsum));
  if constexpr (kCodes) {
    // the V scale of channels 16 db + 4 q4 + (0..3): output = scale * sum p code
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const f4 vs = a.v_quant == kQuantChannel
                        ? *reinterpret_cast<const f4*>(a.v_scale + (int64_t)kvh * D + 16 * db + 4 * q4)
                        : f4{a.v_scale[0], a.v_scale[0], a.v_scale[0], a.v_scale[0]};
      acc[db] *= vs;
    }
  }
  if (pieces > 1) {
    const int64_t pr = ((int64_t)t * a.num_heads + head) * a.chunks;
    if (row_ok) {
      if (q4 == 0) {
        a.part_ml[2 * (pr + piece)] = m;
        a.part_ml[2 * (pr + piece) + 1] = lt;
      }
      float* po = a.part_o + (pr + piece) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *reinterpret_cast<f4*>(po + 16 * db + 4 * q4) = acc[db];
    }
    return;
  }

  const float den = sink_denominator(lt, m, a.use_sink, a.head_sink, head);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  if (row_ok) {
    uint16_t* orow = a.out + (int64_t)t * HD + (int64_t)head * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      uint2 w;
      w.x = (uint32_t)f2h(acc[db][0] * inv) | ((uint32_t)f2h(acc[db][1] * inv) << 16);
      w.y = (uint32_t)f2h(acc[db][2] * inv) | ((uint32_t)f2h(acc[db][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * db + 4 * q4) = w;
    }
  }
}

template <int CT>
void launch_prefill16_cache(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.use_softcap)
    launch_kernel(prefill16_kernel<256, true, CT>, grid, dim3(512), st, a);
  else
    launch_kernel(prefill16_kernel<256, false, CT>, grid, dim3(512), st, a);
}

}  // namespace

hipError_t launch_prefill16(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st) {
  if (head_size != 256) return hipErrorInvalidValue;
  switch (a.cache_dtype) {
    case kCacheI8: launch_prefill16_cache<kCacheI8>(a, grid, st); break;
    case kCacheF8: launch_prefill16_cache<kCacheF8>(a, grid, st); break;
    default: launch_prefill16_cache<kCacheF16>(a, grid, st); break;
  }
  return hipGetLastError();
}

}  // namespace pa
