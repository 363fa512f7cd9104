// Prefill / chunked-prefill attention, 8-wave kernel with 32 query rows per
// wave for the wide head (D = 256) over pools below 4 GiB.
//
// It computes what the kernels in prefill.hip and prefill16.hip compute:
// online-softmax tiled attention (GroupQueryAttention CPU Implementation
// Notes, "Flash Attention Path") with softcap applied to the scaled score
// before masking (PagedAttention -- CUDA Design Document, section 8.5 note),
// causal masking and the window of W positions ending at the query (section
// 4.5), keys addressed one row at a time through the block table.
//
// One workgroup = 8 waves = 256 query rows (token x head-in-group, token
// major) of one kv head, two waves per SIMD.  Each wave owns 32 rows and
// computes, per tile of 32 keys,
//   S^T[key][row] = K[key][:] . Q[row][:]          (v_mfma_f32_32x32x16_f16)
//   O^T[d][row] += V^T[d][key] . P^T[key][row]     (v_mfma_f32_32x32x16_f16)
// so every K or V^T operand read from LDS feeds a 32 x 32 product (half the
// LDS bytes per MFMA of 16-row waves), and every K/V tile staged in LDS is
// shared by 256 rows (half the tile traffic per FLOP of 128-row workgroups).
// The score accumulator is already the B operand of the PV product once the
// keys of a 16-key k-step are taken in the order the accumulator holds them;
// V keeps its row layout and the V^T operand comes from transposing LDS reads.
//
// Tile pipeline: step `it` runs, in one stream of matrix instructions, the QK
// product of tile it and the PV product of tile it - 1 (whose probabilities
// the previous step computed), then the softmax of tile it; K of tile it + 1
// and V of tile it move into LDS during the step (direct buffer loads, 1 KB
// per instruction, issued by one wave of each SIMD; keys that must read as
// zero take an offset past the buffer's end).  One barrier per step.  The two
// waves of a SIMD fill each other's loads and softmax with matrix work.
// Scores are in log2 units with a lazily raised running max.
//
// Quantized pools (PagedAttention -- CUDA Design Document, section 8.5,
// phase 3): the loading waves read each slot's int8 / e4m3fn codes into
// registers and write them into the same LDS slots as fp16 values (every
// such code is an fp16 value).  A per-tensor K scale joins the score scale,
// a per-channel one multiplies Q before its fp16 rounding; the V scale
// multiplies the output accumulator.
#include <type_traits>

#include "prefill_common.h"

namespace pa {

namespace {

struct Rows32Cfg {
  static constexpr int D = 256;
  static constexpr int WAVES = 8;
  static constexpr int ROWS = 256;            // 8 waves x 32 rows
  static constexpr int KT = 32;               // keys per tile
  static constexpr int KS = D / 16;           // QK k-steps (16 channels each)
  static constexpr int DB = D / 32;           // 32-channel output blocks
  static constexpr int CH = D / 8;            // 16-byte chunks per key row
  static constexpr int SLOTS = KT / 2;        // 1 KB slots (two key rows) per tile
  static constexpr int LOADERS = 4;           // waves that move the tiles (one per SIMD)
  static constexpr int DMA = SLOTS / LOADERS; // direct loads per loading wave per tile (K or V)
  static constexpr int KSLOT = 1024 + 16;     // K slot stride (bytes)
  static constexpr int VSLOT = 1024 + 64;     // V slot stride: the 4 rows of a transposing
                                              // read fall 64 bytes apart
  static constexpr int SEGT = 512;            // block-table entries staged per segment
  static constexpr int NPV = 2 * DB;          // PV MFMAs per tile (2 k-steps x DB blocks)
};
static_assert(Rows32Cfg::ROWS == 2 * kPrefillRows, "tiles of two 128-row slots");

// CT: element type of the pools (kCacheF16, or int8 / e4m3fn codes).
template <bool SOFTCAP, int CT>
__global__ __launch_bounds__(512) void prefill32_kernel(const PrefillArgs a) {
  using C = Rows32Cfg;
  constexpr int D = C::D;
  __shared__ __attribute__((aligned(1024))) char K0[C::SLOTS * C::KSLOT];
  __shared__ __attribute__((aligned(1024))) char K1[C::SLOTS * C::KSLOT];
  __shared__ __attribute__((aligned(1024))) char V0[C::SLOTS * C::VSLOT];
  __shared__ __attribute__((aligned(1024))) char V1[C::SLOTS * C::VSLOT];
  __shared__ int32_t s_tbl[C::SEGT];
  __shared__ int sh_b, sh_tile, sh_tb, sh_ql, sh_past;

  const SeqLayout& sl = a.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  __builtin_assume(wave >= 0 && wave < C::WAVES);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const LogicalBlock lb = logical_block();   // XCD-aware order
  const int kvh = lb.y;
  const int g = a.group;
  const int64_t HD = (int64_t)a.num_heads * D;

  if (lb.x == a.tiles * a.chunks) {
    // tokens owned by no request get zero rows (this kv head's columns)
    const int t0 = max(sl.cum[sl.batch], 0);
    const int width = g * C::CH;
    for (int64_t i = tid; i < (int64_t)(sl.tokens - min(t0, sl.tokens)) * width; i += 512) {
      const int t = t0 + (int)(i / width);
      const int cc = (int)(i % width);
      store16(a.out + t * HD + (int64_t)kvh * g * D + 8 * cc, u32x4{0, 0, 0, 0});
    }
    return;
  }

  if (wave == 0) {
    int fb, ft, tb, ql, ps;
    find_tile(sl, g, lb.x / a.chunks, lane, fb, ft, tb, ql, ps, C::ROWS);
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
  // buffers over this kv head's part of each pool (bytes from kbase / vbase on)
  const int64_t pool_bytes = ((sl.num_blocks << shift) * a.kv_heads * D - (int64_t)kvh * D) * 2;
  const int nrec = (int)(uint32_t)min(pool_bytes, (int64_t)0xFFFFFFFF);
  const __amdgpu_buffer_rsrc_t ksrd =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vsrd =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nrec, 0x00020000);
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
  const int R = tile * C::ROWS + wave * 32 + l32;
  const int j = R / g;
  const int hh = R - j * g;
  const bool row_ok = j < q_len && t_begin + j < sl.tokens;
  const int pos = row_ok ? past + j : -1;
  const int t = t_begin + j;
  const int head = kvh * g + hh;

  const TileKeys tk =
      tile_keys(tile, q_len, past, g, a.window, cap, a.chunks, a.piece_tiles, C::ROWS, C::KT);
  const int piece = lb.x - (lb.x / a.chunks) * a.chunks;
  const int pieces = tk.pieces;
  if (piece >= pieces) return;
  const int hi = tk.hi;
  const int lo = tk.lo;
  const int wj0 = min((tile * C::ROWS + wave * 32) / g, q_len - 1);
  const int wj1 = min((tile * C::ROWS + wave * 32 + 31) / g, q_len - 1);
  const int wpos_min = past + wj0;
  const int wpos_max = past + wj1;

  h8 qf[C::KS];   // Q fragments, loaded in the prologue
  f16v acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = kNegInf, lsum = 0.f;

  const int kt_begin = tk.all_begin + piece * tk.per_piece * C::KT;
  const int ntiles = min(tk.per_piece, tk.all_tiles - piece * tk.per_piece);
  int seg_first = -1;      // first block index staged in s_tbl
  bool wg_hole = false;    // some key in [lo, hi) lives in an unmapped block

  // Stage the block-table slice that starts at the block of key `k`.
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
  auto need_segment = [&](int tt) {
    const int last = min(kt_of(tt) + C::KT, hi) - 1;
    return (last >> shift) >= seg_first + C::SEGT;
  };

  // Tile loads: waves 0..3 move every tile, wave w slots w + 4 mi (a wave
  // that issues direct loads stalls while the load pipe drains them, so the
  // other wave of each SIMD keeps the matrix core busy meanwhile); lane i of
  // a slot load moves chunk i % CH of the slot's key row i / CH.  Slot s of a
  // tile holds keys s and s + 16.  The pool row of that key of tile tt, or ~0
  // for a zero row (outside [lo, hi), an unmapped block, or past this
  // workgroup's tiles).
  const bool loader = wave < C::LOADERS;
  auto row_of = [&](int tt, int mi) -> uint32_t {
    const int slot = wave + C::LOADERS * mi;
    const int tau = kt_of(tt) + slot + 16 * (lane / C::CH);
    const bool in = (tt < ntiles) & (tau >= lo) & (tau < hi);
    const int v = s_tbl[in ? (tau >> shift) - seg_first : 0] | (in ? 0 : -1);
    return v < 0 ? ~0u : ((uint32_t)v << shift) | (uint32_t)(tau & bmask);
  };
  const int chunk = lane % C::CH;
  auto dma = [&](uint32_t row, __amdgpu_buffer_rsrc_t srd, char* buf, int slot_bytes, int mi) {
    const uint32_t off = row != ~0u ? (row * tok_stride32 + 8 * chunk) * 2 : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        srd, (__attribute__((address_space(3))) void*)(buf + (wave + C::LOADERS * mi) * slot_bytes),
        16, off, 0, 0, 0);
  };
  // quantized pools: the lane's eight codes of a key row (a zero row reads
  // the zero block: code 0 is +0 in both code types), and their fp16 values
  // written into the lane's 16 bytes of the slot a direct load would fill
  auto load_code = [&](uint32_t row, const char* base) -> u32x2 {
    const int64_t off = row != ~0u ? (int64_t)row * tok_stride32 + 8 * chunk
                                   : reinterpret_cast<const char*>(g_zero_row) - base;
    return *reinterpret_cast<const u32x2*>(base + off);
  };
  auto put_code = [&](u32x2 c, char* buf, int slot_bytes, int mi) {
    *reinterpret_cast<u32x4*>(buf + (wave + C::LOADERS * mi) * slot_bytes + 16 * lane) =
        codes_to_f16<CT>(c);
  };

  // Per-lane parts of the operand addresses (opaque, so each operand read is
  // one base register plus an immediate).  K (A operand of QK): key l32,
  // channels 16 ks + 8 hf.  V^T (A operand of PV) by transposing reads:
  // lane k of each 16-lane group points at 4 channels of one key, lane i then
  // receives channel i of four keys; two reads give the 8 keys of k-step ks
  // that this lane's P operand holds, 16 ks + 8 rr + 4 hf + (0..3).
  int koff = 16 * hf + row_byte<D>(l32, C::KSLOT);
  int voff = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) +
             row_byte<D>(4 * hf + ((lane & 15) >> 2), C::VSLOT);
  asm("" : "+v"(koff), "+v"(voff));
  auto kread = [&](const char* kt, int ks) {
    return *reinterpret_cast<const h8*>(kt + 32 * ks);
  };
  auto vread = [&](const char* vt, int i) {
    const int db = i % C::DB, ks = i / C::DB;
    v4s part2[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      part2[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(vt + row_byte<D>(16 * ks + 8 * rr, C::VSLOT) +
                                                   64 * db));
    h8 v;
    __builtin_memcpy(&v, part2, 16);
    return v;
  };

  // Raw score -> log2-unit logit: scale, or softcap * tanh(scale * s / softcap)
  // with tanh(y) = 1 - 2 / (exp(2y) + 1).
  auto logit = [&](float x) {
    if constexpr (SOFTCAP)
      return a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_fast(x * cap_in2) + 1.0f));
    else
      return x * score_scale;
  };
  // accumulator entry r holds key kt0 + 8 (r / 4) + 4 hf + r % 4 of row l32;
  // keys past the table's capacity (hi is then the capacity) are masked too
  auto full_tile = [&](int kt0) {
    return kt0 >= lo && kt0 + C::KT <= hi && kt0 + C::KT - 1 <= wpos_min &&
           (a.window <= 0 || kt0 >= wpos_max - a.window + 1);
  };
  auto pos_mask = [&](f16v& s, int kt0) {
    const int wlo = a.window > 0 ? pos - a.window + 1 : INT32_MIN;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tau = kt0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      s[r] = ((tau <= pos) & (tau >= wlo) & (tau < hi)) ? s[r] : kNegInf;
    }
  };
  // keys outside [lo, hi) or in an unmapped block (a run of four keys never
  // straddles a block)
  auto hole_mask = [&](f16v& s, int kt0) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int tau0 = kt0 + 8 * rq + 4 * hf;
      const int bi = (tau0 >> shift) - seg_first;
      const int v = bi >= 0 && bi < C::SEGT ? s_tbl[bi] : -1;
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3) {
        const int tau = tau0 + r3;
        if (!(v >= 0 && tau >= lo && tau < hi)) s[4 * rq + r3] = kNegInf;
      }
    }
  };

  // ---- prologue: the table slice, K of tile 0; zero P and V buffer 1, so
  // the first step's PV product (of no tile) adds zeros ----
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  h8 pf[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[k][e] = (_Float16)0.f;

  // One step: QK of tile it (K buffer B) and PV of tile it - 1 (V buffer
  // 1 - B, probabilities in pf), then the softmax of tile it into pf; K of
  // tile it + 1 moves into K buffer 1 - B and V of tile it into V buffer B.
  auto step = [&](int it, auto B) {
    using NB = std::integral_constant<int, 1 - B()>;
    // the staged table slice covers tiles it and it + 1 (this step's loads
    // and masks)
    {
      const int tl = min(it + 1, ntiles - 1);
      if (need_segment(tl)) stage_table(max(kt_of(it), lo));
    }
    if (loader) {
      if constexpr (kCodes) {
        u32x2 cv[C::DMA], ck[C::DMA];
#pragma unroll
        for (int mi = 0; mi < C::DMA; ++mi) {
          cv[mi] = load_code(row_of(it, mi), vcode);
          ck[mi] = load_code(row_of(it + 1, mi), kcode);
        }
#pragma unroll
        for (int mi = 0; mi < C::DMA; ++mi) {
          put_code(cv[mi], vbuf(B), C::VSLOT, mi);
          put_code(ck[mi], kbuf(NB{}), C::KSLOT, mi);
        }
      } else {
        // every slot's table lookup first (a direct load writes LDS, so a
        // lookup after it would wait for the one before), then the loads
        // back to back
        int tv[2 * C::DMA];
#pragma unroll
        for (int q = 0; q < 2 * C::DMA; ++q) {
          const int tt = it + (q & 1);
          const int tau = kt_of(tt) + wave + C::LOADERS * (q >> 1) + 16 * (lane / C::CH);
          const bool in = (tt < ntiles) & (tau >= lo) & (tau < hi);
          tv[q] = s_tbl[in ? (tau >> shift) - seg_first : 0];
        }
        __builtin_amdgcn_sched_barrier(0);   // the lookups go out together
        uint32_t rv[C::DMA], rk[C::DMA];
#pragma unroll
        for (int q = 0; q < 2 * C::DMA; ++q) {
          const int tt = it + (q & 1);
          const int tau = kt_of(tt) + wave + C::LOADERS * (q >> 1) + 16 * (lane / C::CH);
          const bool in = (tt < ntiles) & (tau >= lo) & (tau < hi);
          const uint32_t r = !in || tv[q] < 0 ? ~0u : ((uint32_t)tv[q] << shift) | (uint32_t)(tau & bmask);
          if (q & 1) rk[q >> 1] = r; else rv[q >> 1] = r;
        }
#pragma unroll
        for (int mi = 0; mi < C::DMA; ++mi) dma(rv[mi], vsrd, vbuf(B), C::VSLOT, mi);
#pragma unroll
        for (int mi = 0; mi < C::DMA; ++mi) dma(rk[mi], ksrd, kbuf(NB{}), C::KSLOT, mi);
      }
    }

    // ---- matrix work: QK of tile it interleaved with PV of tile it - 1 ----
    f16v s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
    {
      const char* kt = kbuf(B) + koff;
      const char* vt = vbuf(NB{}) + voff;
      h8 kf = kread(kt, 0), vf[2];
      vf[0] = vread(vt, 0);
      vf[1] = vread(vt, 1);
#pragma unroll
      for (int i = 0; i < C::KS; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[i], s, 0, 0, 0);
        if (i + 1 < C::KS) kf = kread(kt, i + 1);
        const int db = i % C::DB, ks = i / C::DB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i & 1], pf[ks], acc[db], 0, 0, 0);
        if (i + 2 < C::NPV) vf[i & 1] = vread(vt, i + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- softmax of tile it ----
    const int kt0 = kt_of(it);
    if (!full_tile(kt0)) pos_mask(s, kt0);
    if (wg_hole) hole_mask(s, kt0);   // uniform and rare
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = xor32_max(mx);
    mx = mx == kNegInf ? kNegInf : logit(mx);
    // lazy rescale: the running max is only raised when the tile exceeds it
    // by more than kRescaleSlack (probabilities then stay below 2^slack)
    {
      const float mn = mx > m + kRescaleSlack ? mx : m;
      const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
      m = mn;
      lsum *= alpha;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      }
    }
    const float mu = m == kNegInf ? 0.f : m;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = s[r];
      float e;
      if constexpr (SOFTCAP) {
        // cap * tanh(y) - mu = (cap - mu) - 2 cap / (2^t + 1), t = 2y log2(e);
        // a masked score (t = -inf) gets -inf through t * 2^-120
        const float tt = x * cap_in2;
        const float rc = __builtin_amdgcn_rcpf(exp2_fast(tt) + 1.0f);
        e = __builtin_fmaf(tt, 0x1p-120f, __builtin_fmaf(rc, -2.0f * a.cap_out, a.cap_out - mu));
      } else {
        e = __builtin_fmaf(x, score_scale, -mu);
      }
      const float p = exp2_fast(e);
      part += p;
      pf[r >> 3][r & 7] = (_Float16)p;
    }
    lsum += part;
    wait_vmem();       // this wave's tile loads have landed
    __syncthreads();   // ... and everyone's; K buffer B and V buffer 1 - B are free
  };

  // Q fragments (B operand of QK): row l32, channels 16 ks + 8 hf .. +7.
  // Their loads go out with the first K tile's, after the table slice is
  // staged, so the prologue waits on memory twice; chunks that RoPE rotates
  // or a per-channel K scale multiplies are transformed once they landed.
  if (ntiles > 0) stage_table(max(kt_begin, lo));
  const uint16_t* qrow = a.query + (int64_t)t * HD + (int64_t)head * D;
  if (row_ok) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(load16(qrow + 8 * (2 * ks + hf)));
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(u32x4{0, 0, 0, 0});
  }
  auto finish_q = [&]() {
    if (!row_ok || (a.rotary_dim <= 0 && !k_per_channel)) return;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int c = 2 * ks + hf;
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
  };

  if (ntiles > 0) {
    if (loader) {
#pragma unroll
      for (int mi = 0; mi < C::DMA; ++mi) {
        if constexpr (kCodes)
          put_code(load_code(row_of(0, mi), kcode), K0, C::KSLOT, mi);
        else
          dma(row_of(0, mi), ksrd, K0, C::KSLOT, mi);
      }
    }
    for (int i = tid; i < C::SLOTS * C::VSLOT / 16; i += 64 * C::WAVES)
      reinterpret_cast<u32x4*>(V1)[i] = u32x4{0, 0, 0, 0};
    wait_vmem();
    finish_q();
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
      step(it, Buf0{});
      if (it + 1 < ntiles) step(it + 1, Buf1{});
    }
    // PV of the last tile (its V is in buffer (ntiles - 1) % 2; no load is
    // in flight any more, so the buffer may be chosen at run time)
    {
      const char* vt = ((ntiles & 1) ? V0 : V1) + voff;
      h8 vf[2];
      vf[0] = vread(vt, 0);
      vf[1] = vread(vt, 1);
#pragma unroll
      for (int i = 0; i < C::NPV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const int db = i % C::DB, ks = i / C::DB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i & 1], pf[ks], acc[db], 0, 0, 0);
        if (i + 2 < C::NPV) vf[i & 1] = vread(vt, i + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const float lt = xor32_sum(lsum);
  if constexpr (kCodes) {
    // the V scale of channels 32 db + 8 q4 + 4 hf + (0..3): output = scale * sum p code
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * hf;
        const f4 vs = a.v_quant == kQuantChannel
                          ? *reinterpret_cast<const f4*>(a.v_scale + (int64_t)kvh * D + d0)
                          : f4{a.v_scale[0], a.v_scale[0], a.v_scale[0], a.v_scale[0]};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] *= vs[e];
      }
  }
  if (pieces > 1) {
    // ---- one piece of several: store (m, l, unnormalised O) ----
    const int64_t pr = ((int64_t)t * a.num_heads + head) * a.chunks;
    if (row_ok) {
      if (hf == 0) {
        a.part_ml[2 * (pr + piece)] = m;
        a.part_ml[2 * (pr + piece) + 1] = lt;
      }
      float* po = a.part_o + (pr + piece) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f4*>(po + db * 32 + 8 * q4 + 4 * hf) =
              f4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
    }
    return;   // the merge kernel combines the pieces
  }

  // ---- normalise and store: lane (l32, hf) holds channels 32 db + 8 q4 +
  // 4 hf + (0..3) of its row.  The K buffers are free once the loop has
  // ended; each wave passes its rows through 4 KB of them, 64 channels at a
  // time (16-byte slots XOR-swizzled by row), so every store writes whole
  // 128-byte segments of 8 rows.  Lane i stores slot i % 8 of rows
  // i / 8 + 8 k. ----
  const float den = sink_denominator(lt, m, a.use_sink, a.head_sink, head);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  char* stg = (wave < 4 ? K0 : K1) + (wave & 3) * 4096;
  uint16_t* orow_k[4];
  bool rok[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int Rk = tile * C::ROWS + wave * 32 + lane / 8 + 8 * k;
    const int jk = Rk / g;
    rok[k] = jk < q_len && t_begin + jk < sl.tokens;
    orow_k[k] = a.out + (int64_t)(t_begin + jk) * HD + (int64_t)(kvh * g + Rk - jk * g) * D +
                8 * (lane % 8);
  }
#pragma unroll
  for (int rd = 0; rd < C::DB / 2; ++rd) {
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f16v& o = acc[2 * rd + dl];
        uint2 w;
        w.x = (uint32_t)f2h(o[4 * q4 + 0] * inv) | ((uint32_t)f2h(o[4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2h(o[4 * q4 + 2] * inv) | ((uint32_t)f2h(o[4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(stg + l32 * 128 + (((4 * dl + q4) ^ (l32 & 7)) * 16) + 8 * hf) = w;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = lane / 8 + 8 * k;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + rr * 128 + (((lane % 8) ^ (rr & 7)) * 16));
      if (rok[k]) store16(orow_k[k] + 64 * rd, v);
    }
  }
}

}  // namespace

namespace {
template <int CT>
void launch_prefill32_cache(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.use_softcap)
    launch_kernel(prefill32_kernel<true, CT>, grid, dim3(512), st, a);
  else
    launch_kernel(prefill32_kernel<false, CT>, grid, dim3(512), st, a);
}
}  // namespace

hipError_t launch_prefill32(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st) {
  if (head_size != Rows32Cfg::D || !a.pool32) return hipErrorInvalidValue;
  switch (a.cache_dtype) {
    case kCacheI8: launch_prefill32_cache<kCacheI8>(a, grid, st); break;
    case kCacheF8: launch_prefill32_cache<kCacheF8>(a, grid, st); break;
    default: launch_prefill32_cache<kCacheF16>(a, grid, st); break;
  }
  return hipGetLastError();
}

}  // namespace pa
