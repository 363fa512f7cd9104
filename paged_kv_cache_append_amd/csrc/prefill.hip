// Prefill / chunked-prefill attention over the paged pool with fp16 MFMA.
//
// Online-softmax tiled attention (GroupQueryAttention CPU Implementation
// Notes, "Flash Attention Path": QK on a KV block, causal + local-window
// masking, running max/sum with exp(m_old - m_new) rescale, fused SV
// accumulate, 1/l at the end) with softcap applied to the scaled score before
// masking (PagedAttention -- CUDA Design Document, section 8.5 note) and the
// window of W positions ending at the query (section 4.5).  Tiles address the
// pool one key row at a time through the block table, so a tile may straddle
// pages of any power-of-two block size (the straddling limit of section 18.1
// does not arise).
//
// One workgroup = 4 waves = 128 query rows of one kv head; a row is a (query
// token, head-in-group) pair, token-major, so every K/V tile staged in LDS is
// shared by all heads of the group.  Each wave owns 32 rows and computes
//   S^T[key][row] = K[key][:] . Q[row][:]          (v_mfma_f32_32x32x16_f16)
// so that the score accumulator already has the B-operand layout of
//   O^T[d][row] += V^T[d][key] . P^T[key][row]
// and the probabilities go from registers to the MFMA without an LDS round
// trip.  K and V tiles of 64 keys move from the pool straight into LDS with
// direct loads (no staging registers), two buffers each; V keeps its natural
// row layout and the V^T operand comes from transposing LDS reads.  The tile
// loop is software-pipelined with K one tile ahead of V: while the QK
// product of the next tile runs on the matrix cores, the vector ALU computes
// the current tile's probabilities and issues the next loads, and while the
// PV product of the current tile runs, it finishes the probabilities and
// takes the next tile's row maximum.  One barrier per tile.  The block-table
// slice of the workgroup's key range is staged in LDS.  Scores are in log2
// units; the running max is shared by the two lanes of a row with one lane
// swap per tile and is only raised when a tile exceeds it by more than 8
// (lazy rescale).
//
// Quantized pools (PagedAttention -- CUDA Design Document, section 8.5,
// phase 3, here for multi-token requests too): each lane loads its eight
// codes of a key row into a register instead of the direct load, and writes
// them as eight fp16 values (int8 and e4m3fn values are exact in fp16) into
// the same LDS slot once the step's matrix work is done; the buffers written
// are the ones no wave reads during the step, as with the direct loads.  A
// per-tensor K scale joins the score scale, a per-channel one multiplies Q
// (then rounded to fp16); the V scale multiplies the output accumulator.
#include <type_traits>

#include "prefill_common.h"

namespace pa {

namespace {

template <int D>
struct PrefillCfg {
  static constexpr int ROWS = kPrefillRows;  // 128 rows = 4 waves x 32
  static constexpr int KT = 64;              // keys per tile
  static constexpr int KS = D / 16;          // QK k-steps over the head dim
  static constexpr int DB = D / 32;          // 32-channel output blocks
  static constexpr int CH = D / 8;           // 16-byte chunks per key row
  static constexpr int RPS = 64 / CH;        // key rows per 1 KB slot (one direct load)
  static constexpr int NS = 32 / RPS;        // slots per 32-key block
  static constexpr int SLOTS = KT / RPS;     // slots per tile
  static constexpr int KSLOT = 1024 + 16;    // K slot stride (bytes): rows read together
                                             // by 8 lanes fall 16 bytes apart
  static constexpr int VSLOT = 1024 + 64;    // V slot stride: the 4 rows of a transposing
                                             // read fall 64 bytes apart
  static constexpr int DMA = SLOTS / 4;      // direct loads per wave per tile (K or V)
  static constexpr int SEGT = 512;           // block-table entries staged per segment
  static constexpr int PIPE = KS < 2 ? KS : 2;   // operand reads in flight (k-steps)
};

// BUF: the tiles move by buffer loads with an LDS destination and 32-bit byte
// offsets (each cache smaller than 4 GiB), otherwise by global loads with an
// LDS destination.  The buffer form leaves the compiler free to wait on
// individual LDS operand reads; with the global form it waits on all of them.
//
// CT: element type of the pools (kCacheF16, or int8 / e4m3fn codes, which
// take the register path above; BUF is then unused).
template <int D, bool SOFTCAP, bool BUF, int CT>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs a) {
  using C = PrefillCfg<D>;
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
  __builtin_assume(wave >= 0 && wave < 4);
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
    for (int64_t i = tid; i < (int64_t)(sl.tokens - min(t0, sl.tokens)) * width; i += 256) {
      const int t = t0 + (int)(i / width);
      const int cc = (int)(i % width);
      store16(a.out + t * HD + (int64_t)kvh * g * D + 8 * cc, u32x4{0, 0, 0, 0});
    }
    return;
  }

  // Map this workgroup to (request, tile) over requests with q_len >= 2.
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
  const int b = __builtin_amdgcn_readfirstlane(sh_b);          // uniform per workgroup
  if (b < 0) return;
  const int tile = __builtin_amdgcn_readfirstlane(sh_tile);

  const int t_begin = __builtin_amdgcn_readfirstlane(sh_tb);
  const int q_len = __builtin_amdgcn_readfirstlane(sh_ql);
  const int past = __builtin_amdgcn_readfirstlane(sh_past);
  const int cap = sl.maxblk << sl.block_shift;
  const int shift = sl.block_shift;
  const int bmask = (1 << shift) - 1;
  const int32_t* bt = sl.block_table + (int64_t)b * sl.maxblk;
  const int64_t tok_stride = (int64_t)a.kv_heads * D;
  const uint32_t tok_stride32 = (uint32_t)tok_stride;   // Hkv * D < 2^24
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

  // key range of the whole tile, and of this wave's rows (fast path)
  const TileKeys tk = tile_keys(tile, q_len, past, g, a.window, cap, a.chunks, a.piece_tiles);
  const int piece = lb.x - (lb.x / a.chunks) * a.chunks;
  const int pieces = tk.pieces;
  if (piece >= pieces) return;
  const int hi = tk.hi;
  const int lo = tk.lo;
  const int wj0 = min((tile * C::ROWS + wave * 32) / g, q_len - 1);
  const int wj1 = min((tile * C::ROWS + wave * 32 + 31) / g, q_len - 1);
  const int wpos_min = past + wj0;
  const int wpos_max = past + wj1;

  // Q fragments (B operand): row l32, channels 16*ks + 8*hf .. +7
  // all chunk loads first (one memory round trip), then the chunks that
  // RoPE rotates or a per-channel K scale multiplies
  h8 qf[C::KS];
  const uint16_t* qrow = a.query + (int64_t)t * HD + (int64_t)head * D;
  if (row_ok) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(load16(qrow + 8 * (2 * ks + hf)));
  } else {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = as_h8(u32x4{0, 0, 0, 0});
  }
  if (row_ok && (a.rotary_dim > 0 || k_per_channel)) {
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
  }
  // Let the query loads land here: otherwise the first MFMA of every tile
  // would wait for them with a full vmcnt(0), i.e. also for the next tile's
  // loads that were just issued.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  f16v acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = kNegInf, lsum = 0.f;

  // This workgroup's piece of the key range: the tile's key tiles split into
  // a.chunks nearly equal runs (pieces past the end have nothing to do).
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
    for (int i = tid; i < C::SEGT; i += 256) {
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
  auto kt_of = [&](int t) { return kt_begin + t * C::KT; };

  // Key rows this wave moves for key tile t (wave w fills slots w, w + 4,
  // ...; lane i of a slot load moves chunk i % CH of key row i / CH of the
  // slot) and their pool blocks: -1 for keys outside [lo, hi), in an unmapped
  // block, or in a tile past this workgroup's range (those read a zero row).
  // Branch-free, so it can share a scheduling region with the matrix work.
  auto lookup = [&](int t, int (&tau)[C::DMA], int (&blk)[C::DMA]) {
    const int kt0 = kt_of(t);
    const bool valid = t < ntiles;
#pragma unroll
    for (int mi = 0; mi < C::DMA; ++mi) {
      const int slot = wave + 4 * mi;
      tau[mi] = kt0 + (slot / C::NS) * 32 + (slot % C::NS) + C::NS * (lane / C::CH);
      // bitwise tests and an OR with 0 / -1 (not a select of the loaded
      // value) keep this free of branches
      const bool in = valid & (tau[mi] >= lo) & (tau[mi] < hi);
      const int v = s_tbl[in ? (tau[mi] >> shift) - seg_first : 0];
      blk[mi] = v | (in ? 0 : -1);
    }
  };
  // The same for one load: the pool row (block * block_size + offset) of the
  // key row this lane moves with load mi of tile t, or ~0 for a zero row (pools
  // hold fewer than 2^32 rows).
  auto row_of = [&](int t, int mi) -> uint32_t {
    const int slot = wave + 4 * mi;
    const int tau = kt_of(t) + (slot / C::NS) * 32 + (slot % C::NS) + C::NS * (lane / C::CH);
    const bool in = (t < ntiles) & (tau >= lo) & (tau < hi);
    const int v = s_tbl[in ? (tau >> shift) - seg_first : 0] | (in ? 0 : -1);
    return v < 0 ? ~0u : ((uint32_t)v << shift) | (uint32_t)(tau & bmask);
  };
  const int chunk = lane % C::CH;
  const uint16_t* zrow = g_zero_row + 8 * chunk;
  // quantized pools: this lane's eight codes of a key row (a zero row reads
  // the zero block: code 0 is +0 in both code types), and their fp16 values
  // written into the lane's 16 bytes of an LDS slot
  auto load_codes = [&](uint32_t row, const char* base) -> u32x2 {
    const int64_t off = row != ~0u ? (int64_t)row * tok_stride + 8 * chunk
                                   : reinterpret_cast<const char*>(g_zero_row) - base;
    return *reinterpret_cast<const u32x2*>(base + off);
  };
  auto put_codes = [&](u32x2 c, char* buf, int slot_bytes, int mi) {
    const int slot = wave + 4 * mi;
    *reinterpret_cast<u32x4*>(buf + slot * slot_bytes + 16 * lane) = codes_to_f16<CT>(c);
  };
  auto issue_row = [&](uint32_t row, const uint16_t* base, char* buf, int slot_bytes, int mi) {
    const int slot = wave + 4 * mi;
    if constexpr (kCodes) {
      put_codes(load_codes(row, base == vbase ? vcode : kcode), buf, slot_bytes, mi);
    } else if constexpr (BUF) {
      // a zero row: an offset past the buffer's end reads zeros
      const uint32_t off = row != ~0u ? (row * tok_stride32 + 8 * chunk) * 2 : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          base == vbase ? vsrd : ksrd,
          (__attribute__((address_space(3))) void*)(buf + slot * slot_bytes), 16, off, 0, 0, 0);
    } else {
      // one source pointer, base + a selected element offset (a select between
      // two pointers makes the compiler split the load in two exec-masked halves)
      const int64_t off =
          row != ~0u ? (int64_t)((uint64_t)row * tok_stride32 + 8 * chunk) : zrow - base;
      dma16(base + off, buf + slot * slot_bytes);
    }
  };
  auto issue_one = [&](int tau, int blk, const uint16_t* base, char* buf, int slot_bytes,
                       int mi) {
    const uint32_t row = blk < 0 ? ~0u : ((uint32_t)blk << shift) | (uint32_t)(tau & bmask);
    issue_row(row, base, buf, slot_bytes, mi);
  };
  auto issue = [&](const int (&tau)[C::DMA], const int (&blk)[C::DMA], const uint16_t* base,
                   char* buf, int slot_bytes) {
#pragma unroll
    for (int mi = 0; mi < C::DMA; ++mi) issue_one(tau[mi], blk[mi], base, buf, slot_bytes, mi);
  };
  // the last key tile a staged table slice must cover is within reach
  auto need_segment = [&](int t) {
    const int last = min(kt_of(t) + C::KT, hi) - 1;
    return (last >> shift) >= seg_first + C::SEGT;
  };

  // S^T = K . Q^T for two 32-key blocks of the tile in K buffer B.  The two
  // blocks alternate so consecutive MFMAs are independent; operand reads run
  // PIPE k-steps ahead (their order is fixed by the caller's schedule).
  // Per-lane parts of the operand addresses, made opaque so every operand
  // read is one variable base plus a constant: the compiler otherwise splits
  // them into long address chains whose reads lose the information that they
  // cannot overlap the loads streaming into the other buffers (and then wait
  // for those loads).  row_byte(c + x) = row_byte(c) + row_byte(x) for c a
  // multiple of 8 and x < 8.
  int koff = 16 * hf + row_byte<D>(l32, C::KSLOT);
  int voff = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) +
             row_byte<D>(4 * hf + ((lane & 15) >> 2), C::VSLOT);
  asm("" : "+v"(koff), "+v"(voff));

  auto qk = [&](auto B, f16v (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    const char* kt = kbuf(B) + koff;
    auto kread = [&](int ks, int kb) {
      return *reinterpret_cast<const h8*>(kt + row_byte<D>(kb * 32, C::KSLOT) + 32 * ks);
    };
    h8 kf[C::PIPE][2];
#pragma unroll
    for (int i = 0; i < C::PIPE; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[i][kb] = kread(i, kb);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % C::PIPE][kb], qf[ks], s[kb], 0, 0, 0);
        if (ks + C::PIPE < C::KS) kf[ks % C::PIPE][kb] = kread(ks + C::PIPE, kb);
      }
    }
  };

  // Raw score -> log2-unit logit: scale, or softcap * tanh(scale * s / softcap)
  // with tanh(y) = 1 - 2 / (exp(2y) + 1) (exact limits +-1 for large |y|).
  auto logit = [&](float x) {
    if constexpr (SOFTCAP)
      return a.cap_out * (1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_fast(x * cap_in2) + 1.0f));
    else
      return x * score_scale;
  };
  // A row's tile maximum in log2 units (scale and softcap are monotone, so
  // the maximum is taken on raw scores); the row's two lanes agree.
  auto tile_max = [&](const f16v (&s)[2]) {
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      mq[q] = fmaxf(fmaxf(s[q >> 1][8 * (q & 1)], s[q >> 1][8 * (q & 1) + 1]),
                    fmaxf(s[q >> 1][8 * (q & 1) + 2], s[q >> 1][8 * (q & 1) + 3]));
#pragma unroll
      for (int r = 4; r < 8; ++r) mq[q] = fmaxf(mq[q], s[q >> 1][8 * (q & 1) + r]);
    }
    const float mx = xor32_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
    return mx == kNegInf ? kNegInf : logit(mx);
  };
  // Keys outside the row's causal window, or past the table's capacity (hi
  // is then the capacity); accumulator entry r of block kb holds key
  // kt0 + 32 kb + 8 (r / 4) + 4 hf + r % 4.
  auto full_tile = [&](int kt0) {
    return kt0 >= lo && kt0 + C::KT <= hi && kt0 + C::KT - 1 <= wpos_min &&
           (a.window <= 0 || kt0 >= wpos_max - a.window + 1);
  };
  auto pos_mask = [&](f16v (&s)[2], int kt0) {
    const int wlo = a.window > 0 ? pos - a.window + 1 : INT32_MIN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tau = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        s[kb][r] = ((tau <= pos) & (tau >= wlo) & (tau < hi)) ? s[kb][r] : kNegInf;
      }
  };
  // Keys outside [lo, hi) or in an unmapped block (only when the key range
  // has a hole; the staged table slice still covers the tile).  A run of four
  // keys never straddles a block.
  auto hole_mask = [&](f16v (&s)[2], int kt0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int tau0 = kt0 + kb * 32 + 8 * rq + 4 * hf;
        const int bi = (tau0 >> shift) - seg_first;
        const int v = bi >= 0 && bi < C::SEGT ? s_tbl[bi] : -1;
#pragma unroll
        for (int r3 = 0; r3 < 4; ++r3) {
          const int tau = tau0 + r3;
          if (!(v >= 0 && tau >= lo && tau < hi)) s[kb][4 * rq + r3] = kNegInf;
        }
      }
  };

  // Probabilities p = 2^(logit - mu) of scores f0 .. f0 + n - 1 (f = 16 kb +
  // r) of a tile, into the fp16 B operand of the PV product (k-step ks covers
  // accumulator rows 8 (ks & 1) .. +7 of 32-key block ks / 2); their sums
  // accumulate in part.  A masked score (-inf) gives 0.
  auto softmax_part = [&](const f16v (&s)[2], float mu, h8 (&pf)[4], float (&part)[4], int f0,
                          int n) {
#pragma unroll
    for (int f = f0; f < f0 + n; ++f) {
      const int kb = f >> 4, r = f & 15;
      const float x = s[kb][r];
      float e;
      if constexpr (SOFTCAP) {
        // cap * tanh(y) - mu = (cap - mu) - 2 cap / (2^t + 1), t = 2y log2(e);
        // a masked score (t = -inf) gets -inf through t * 2^-120, which is
        // negligible for any finite t
        const float t = x * cap_in2;
        const float r = __builtin_amdgcn_rcpf(exp2_fast(t) + 1.0f);
        e = __builtin_fmaf(t, 0x1p-120f, __builtin_fmaf(r, -2.0f * a.cap_out, a.cap_out - mu));
      } else {
        e = __builtin_fmaf(x, score_scale, -mu);
      }
      const float p = exp2_fast(e);
      part[r & 3] += p;
      pf[2 * kb + (r >> 3)][r & 7] = (_Float16)p;
    }
  };

  // O^T += V^T . P^T (region B of a step) takes the V^T operand from
  // transposing LDS reads: lane k of each 16-lane group points at 4 channels
  // of one key; lane i then receives channel i of four keys.  Two reads give
  // the 8 keys of k-step ks that the P operand of this lane holds:
  // 16 ks + 8 rr + 4 hf + (0..3), rr = 0, 1.
  constexpr int NV = 4 * C::DB;

  // ---- prologue: K and V of tile 0 and K of tile 1, then tile 0's scores ----
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  f16v sA[2], sB[2];
  float mxA = kNegInf, mxB = kNegInf;
  if (ntiles > 0) {
    stage_table(max(kt_begin, lo));
    int t0[C::DMA], b0[C::DMA], t1[C::DMA], b1[C::DMA];
    lookup(0, t0, b0);
    lookup(1, t1, b1);
    issue(t0, b0, kbase, K0, C::KSLOT);
    issue(t0, b0, vbase, V0, C::VSLOT);
    issue(t1, b1, kbase, K1, C::KSLOT);
    wait_vmem();
    __syncthreads();
    qk(Buf0{}, sA);
    pipeline_order<2 * C::PIPE, 2 * C::KS, 1>();
    if (!full_tile(kt_of(0))) pos_mask(sA, kt_of(0));
    mxA = tile_max(sA);
    __syncthreads();   // K buffer 0 is refilled by the first step
  }

  // One step: the softmax and PV product of key tile `it` (scores in s_cur,
  // V in buffer B) while tile it + 1's scores are computed (K in buffer 1 - B)
  // and the loads of tile it + 1's V and tile it + 2's K stream in.  The
  // softmax, the load issue and the QK product form one scheduling region,
  // as do the PV product and the next tile's row maximum, so the vector ALU
  // and the matrix cores work at the same time.
  auto step = [&](int it, auto B, f16v (&s_cur)[2], f16v (&s_next)[2], float& mx_cur,
                  float& mx_next) {
    using NB = std::integral_constant<int, 1 - B()>;
    if (wg_hole) {   // uniform and rare
      hole_mask(s_cur, kt_of(it));
      mx_cur = tile_max(s_cur);
    }
    // lazy rescale: the running max is only raised when the tile exceeds it
    // by more than kRescaleSlack (probabilities then stay below 2^slack)
    {
      const float mn = mx_cur > m + kRescaleSlack ? mx_cur : m;
      const float alpha = mn == m ? 1.0f : exp2_fast(m - mn);
      m = mn;
      lsum *= alpha;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
    }
    const float mu = m == kNegInf ? 0.f : m;
    {
      const int tl = min(it + 2, ntiles - 1);
      if (tl > it && need_segment(tl)) stage_table(max(kt_of(it + 1), lo));
    }

    // ---- region A: QK of tile it + 1, with the softmax of tile it and the
    // loads of tile it + 1's V and tile it + 2's K spread over its k-steps
    // (2 DMA = KS direct loads, one per k-step).  Each k-step is fenced so
    // the vector work stays between the matrix instructions. ----
    h8 pf[4];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    u32x2 codes[kCodes ? C::KS : 1];   // quantized pools: this step's loads, written at its end
    {
      // load j of the step: tile it + 1's V (j < DMA), then tile it + 2's K;
      // its table lookup is issued one k-step before the load
      auto row_j = [&](int j) { return j < C::DMA ? row_of(it + 1, j) : row_of(it + 2, j - C::DMA); };
      uint32_t row_next = row_j(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s_next[kb][i] = 0.f;
      const char* kt = kbuf(NB{}) + koff;
      auto kread = [&](int ks, int kb) {
        return *reinterpret_cast<const h8*>(kt + row_byte<D>(kb * 32, C::KSLOT) + 32 * ks);
      };
      h8 kf[C::PIPE][2];
#pragma unroll
      for (int i = 0; i < C::PIPE; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kf[i][kb] = kread(i, kb);
      // probabilities of the tile's first 16-key k-step (pf[0], scores 0..7
      // of this lane) here, in pairs at k-steps 0, KS/4, KS/2, 3KS/4; the other
      // three quarters are computed in region B during the PV MFMAs of the
      // quarter before
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks % C::PIPE][kb], qf[ks], s_next[kb], 0, 0, 0);
          if (ks + C::PIPE < C::KS) kf[ks % C::PIPE][kb] = kread(ks + C::PIPE, kb);
        }
        const uint32_t row = row_next;
        if (ks + 1 < C::KS) row_next = row_j(ks + 1);
        if constexpr (kCodes)
          codes[ks] = load_codes(row, ks < C::DMA ? vcode : kcode);
        else if (ks < C::DMA)
          issue_row(row, vbase, vbuf(NB{}), C::VSLOT, ks);
        else
          issue_row(row, kbase, kbuf(B), C::KSLOT, ks - C::DMA);
        if (ks % (C::KS / 4) == 0) {
          softmax_part(s_cur, mu, pf, part, 2 * (ks / (C::KS / 4)), 2);
          // anchor: the compiler would otherwise sink the exponentials down
          // to their use in region B
          asm volatile("" ::"v"(part[0]), "v"(part[1]), "v"(part[2]), "v"(part[3]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- region B: PV of tile it, with tile it + 1's row maximum spread
    // over its MFMAs ----
    {
      const char* vt = vbuf(B) + voff;
      auto vread = [&](int i) {
        const int db = i % C::DB, ks = i / C::DB;
        v4s part2[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          part2[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s*)(
                  vt + row_byte<D>(16 * ks + 8 * rr, C::VSLOT) + 64 * db));
        h8 v;
        __builtin_memcpy(&v, part2, 16);
        return v;
      };
      h8 vf[2 * C::PIPE];
#pragma unroll
      for (int i = 0; i < 2 * C::PIPE; ++i) vf[i] = vread(i);
      constexpr int MPC = 32 / NV > 0 ? 32 / NV : 1;   // max operands per MFMA
      float mxr = kNegInf;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        const int db = i % C::DB, ks = i / C::DB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i % (2 * C::PIPE)], pf[ks], acc[db], 0, 0, 0);
        if (i + 2 * C::PIPE < NV) vf[i % (2 * C::PIPE)] = vread(i + 2 * C::PIPE);
        // pf[ks + 1] in pairs at MFMAs DB/4 apart
        if (ks + 1 < 4) {
#pragma unroll
          for (int pr = 0; pr < 4; ++pr)
            if ((pr * C::DB) / 4 == db) softmax_part(s_cur, mu, pf, part, 8 * (ks + 1) + 2 * pr, 2);
        }
#pragma unroll
        for (int f = i * MPC; f < (i + 1) * MPC && f < 32; ++f)
          mxr = fmaxf(mxr, s_next[f >> 4][f & 15]);
        asm volatile("" ::"v"(mxr), "v"(part[0]), "v"(part[1]), "v"(part[2]), "v"(part[3]));
      }
      __builtin_amdgcn_sched_barrier(0);
      lsum += (part[0] + part[1]) + (part[2] + part[3]);
      mxr = xor32_max(mxr);
      mx_next = mxr == kNegInf ? kNegInf : logit(mxr);
    }
    if (it + 1 < ntiles && !full_tile(kt_of(it + 1))) {   // diagonal / window-edge tiles
      pos_mask(s_next, kt_of(it + 1));
      mx_next = tile_max(s_next);
    }
    if constexpr (kCodes) {
      // tile it + 1's V into buffer 1 - B and tile it + 2's K into buffer B:
      // neither is read by any wave during this step
#pragma unroll
      for (int j = 0; j < C::KS; ++j) {
        if (j < C::DMA)
          put_codes(codes[j], vbuf(NB{}), C::VSLOT, j);
        else
          put_codes(codes[j], kbuf(B), C::KSLOT, j - C::DMA);
      }
    }
    wait_vmem();        // this wave's loads have landed
    __syncthreads();    // ... and everyone's; buffers B (V) and 1 - B (K) are free
  };

  for (int it = 0; it < ntiles; it += 2) {
    step(it, Buf0{}, sA, sB, mxA, mxB);
    if (it + 1 < ntiles) step(it + 1, Buf1{}, sB, sA, mxB, mxA);
  }

  const float lt = xor32_sum(lsum);
  if constexpr (kCodes) {
    // the V scale of channels db * 32 + 8 q4 + 4 hf + (0..3): output = scale * sum p code
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

  // ---- normalise and store ----
  const float den = sink_denominator(lt, m, a.use_sink, a.head_sink, head);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  if (row_ok) {
    uint16_t* orow = a.out + (int64_t)t * HD + (int64_t)head * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = db * 32 + 8 * q4 + 4 * hf;
        uint2 w;
        w.x = (uint32_t)f2h(acc[db][4 * q4 + 0] * inv) | ((uint32_t)f2h(acc[db][4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2h(acc[db][4 * q4 + 2] * inv) | ((uint32_t)f2h(acc[db][4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    }
  }
}

// One row of a tile cut into pieces: combine its pieces' partials.
template <int D>
__device__ __forceinline__ void merge_row(const PrefillArgs& a, const TileKeys& tk, int t_begin,
                                          int q_len, int R, int tid) {
  const SeqLayout& sl = a.s;
  const int g = a.group;
  const int j = R / g;
  if (j >= q_len || t_begin + j >= sl.tokens) return;
  const int t = t_begin + j;
  const int head = blockIdx.y * g + (R - j * g);
  const int64_t pr = ((int64_t)t * a.num_heads + head) * a.chunks;
  float w[kPrefillChunks];
  float mm = kNegInf, ll = 0.f;
#pragma unroll
  for (int c = 0; c < kPrefillChunks; ++c)
    if (c < tk.pieces) mm = fmaxf(mm, a.part_ml[2 * (pr + c)]);
#pragma unroll
  for (int c = 0; c < kPrefillChunks; ++c) {
    w[c] = c < tk.pieces && mm != kNegInf ? exp2_fast(a.part_ml[2 * (pr + c)] - mm) : 0.f;
    if (c < tk.pieces) ll += w[c] * a.part_ml[2 * (pr + c) + 1];
  }
  ll = sink_denominator(ll, mm, a.use_sink, a.head_sink, head);
  const float inv = ll > 0.f ? 1.0f / ll : 0.f;
  uint16_t* orow = a.out + (int64_t)t * a.num_heads * D + (int64_t)head * D;
#pragma unroll 4
  for (int d0 = (tid & 1) * (D / 2); d0 < (tid & 1) * (D / 2) + D / 2; d0 += 4) {
    f4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kPrefillChunks; ++c)
      if (c < tk.pieces) o += w[c] * *reinterpret_cast<const f4*>(a.part_o + (pr + c) * D + d0);
    uint2 v;
    v.x = (uint32_t)f2h(o[0] * inv) | ((uint32_t)f2h(o[1] * inv) << 16);
    v.y = (uint32_t)f2h(o[2] * inv) | ((uint32_t)f2h(o[3] * inv) << 16);
    *reinterpret_cast<uint2*>(orow + d0) = v;
  }
}

// Combine the pieces of every prefill tile cut into several: one workgroup
// per (tile slot, kv head); thread pairs own a row, each half of its channels.
// o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c, with M = max_c m_c
// (GroupQueryAttention CPU Implementation Notes, "Flash Decoding" merge).
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a) {
  __shared__ int sh_b, sh_tile;
  const SeqLayout& sl = a.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = a.group;
  if (tid < 64) {
    int fb, ft;
    find_tile(sl, g, blockIdx.x, lane, fb, ft, a.tile_rows);
    if (lane == 0) {
      sh_b = fb;
      sh_tile = ft;
    }
  }
  __syncthreads();
  const int b = __builtin_amdgcn_readfirstlane(sh_b);
  if (b < 0) return;
  const int tile = __builtin_amdgcn_readfirstlane(sh_tile);
  const int t_begin = sl.cum[b];
  const int q_len = sl.cum[b + 1] - t_begin;
  const TileKeys tk = tile_keys(tile, q_len, sl.past[b], g, a.window, sl.maxblk << sl.block_shift,
                                a.chunks, a.piece_tiles, a.tile_rows, a.key_tile);
  if (tk.pieces <= 1) return;
  // a tile slot of tile_rows rows: thread pairs take rows tid / 2, + 128, ...
  for (int r0 = 0; r0 < a.tile_rows; r0 += 128)
    merge_row<D>(a, tk, t_begin, q_len, tile * a.tile_rows + r0 + (tid >> 1), tid);
}

template <int D, bool BUF, int CT>
void launch_variant(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.use_softcap)
    launch_kernel(prefill_kernel<D, true, BUF, CT>, grid, dim3(256), st, a);
  else
    launch_kernel(prefill_kernel<D, false, BUF, CT>, grid, dim3(256), st, a);
}
// quantized pools take the register path; fp16 pools the buffer-form direct
// loads when each cache is below 4 GiB (never instantiated for D = 256, whose
// small pools take the 8-wave kernel)
template <int D>
void launch_variant(const PrefillArgs& a, dim3 grid, hipStream_t st) {
  if (a.cache_dtype == kCacheI8)
    launch_variant<D, false, kCacheI8>(a, grid, st);
  else if (a.cache_dtype == kCacheF8)
    launch_variant<D, false, kCacheF8>(a, grid, st);
  else if constexpr (D != 256) {
    if (a.pool32)
      launch_variant<D, true, kCacheF16>(a, grid, st);
    else
      launch_variant<D, false, kCacheF16>(a, grid, st);
  } else {
    launch_variant<D, false, kCacheF16>(a, grid, st);
  }
}

}  // namespace

hipError_t launch_prefill_merge(const PrefillArgs& a, int head_size, hipStream_t st) {
  const dim3 grid(a.tiles, a.kv_heads);
  switch (head_size) {
    case 64: launch_kernel(prefill_merge_kernel<64>, grid, dim3(256), st, a); break;
    case 128: launch_kernel(prefill_merge_kernel<128>, grid, dim3(256), st, a); break;
    case 256: launch_kernel(prefill_merge_kernel<256>, grid, dim3(256), st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st) {
  switch (head_size) {
    case 64: launch_variant<64>(a, grid, st); break;
    case 128: launch_variant<128>(a, grid, st); break;
    case 256:
      if (a.rows32) return launch_prefill32(a, head_size, grid, st);
      if (a.rows16) return launch_prefill16(a, head_size, grid, st);
      launch_variant<256>(a, grid, st);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
