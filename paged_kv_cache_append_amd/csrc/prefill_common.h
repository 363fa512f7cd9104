// Pieces shared by the prefill kernels (prefill.hip: 4 waves of 32 rows,
// prefill16.hip: 8 waves of 16 rows): tile layout in LDS, direct loads,
// tile -> request mapping, key ranges of a tile, lane-swap reductions.
#pragma once

#include "pa_device.h"

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 units
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Tile layout in LDS: key row r (0..63) of the tile lives in slot
// (r / 32) * NS + (r % NS) at row position ((r % 32) / NS) within the slot;
// a slot is one contiguous 1 KB direct load plus padding, and every operand
// address is a base register plus an immediate offset.
template <int D>
__device__ __forceinline__ int row_byte(int r, int slot_bytes) {
  constexpr int NS = D / 16;   // slots per 32-key block (a 1 KB slot holds 512 / D rows)
  return ((r >> 5) * NS + (r % NS)) * slot_bytes + ((r & 31) / NS) * (2 * D);
}

// Workgroup placement: the hardware deals consecutive linear workgroup ids to
// the chip's 8 XCDs in turn, each XCD with its own L2.  This maps the linear
// id of a workgroup to a logical id such that the workgroups placed on one XCD
// take one contiguous range of logical ids (a bijection for any total), so
// tiles that read the same K/V tiles share that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int linear, int total) {
  constexpr int kXcds = 8;
  const int q = total / kXcds, r = total % kXcds;
  const int xcd = linear % kXcds, k = linear / kXcds;
  return xcd * q + min(xcd, r) + k;
}
// (x, y) of this workgroup in the logical order
struct LogicalBlock {
  int x, y;
};
__device__ __forceinline__ LogicalBlock logical_block() {
  const int linear = blockIdx.x + blockIdx.y * gridDim.x;
  const int l = xcd_logical_id(linear, gridDim.x * gridDim.y);
  return LogicalBlock{l % (int)gridDim.x, l / (int)gridDim.x};
}

// Source of the rows that must read as zero (never written).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[256];

__device__ __forceinline__ void dma16(const uint16_t* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// vmcnt(0), no wait on the LDS/scalar counter
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Scheduling order of a block of N MFMAs fed by RPM LDS reads each: the
// reads of the first AHEAD MFMAs, then one MFMA per further group of reads,
// then the remaining MFMAs, so every operand is requested AHEAD MFMA issue
// slots before its use.  The compiler otherwise pulls each read down next to
// its MFMA to save registers.
template <int AHEAD, int N, int RPM>
__device__ __forceinline__ void pipeline_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD * RPM, 0);   // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);         // DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Tile slot -> (request b, tile) over requests with q_len >= 2, tiles of
// `rows` rows (token x head-in-group) each.  b = -1 past the last tile.
// Called by a whole wave; the results are the same in every lane.
//
// Order (the hardware starts the workgroups of an XCD in slot order, each on
// the next CU that frees): request b is in group S_b / kGroupTiles, S_b being
// the number of tiles of the requests before it, so a group spans at least
// the CUs of one XCD.  A group's slots hold its tiles by rank -- rank 0 is
// every request's last (longest) tile, then rank 1, ..., requests in order
// within a rank -- so long and short tiles pair up on the CUs, and the
// requests of a group walk their keys together.  When all tiles fit one XCD's
// CUs at once, no tile waits for another to finish and every request is a
// group of its own (its tiles longest first): the tiles of one request then
// start together, and a decode running beside a small prefill keeps more of
// the chip.
constexpr int kGroupTiles = 32;   // CUs per XCD
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// The request's first token, query length and past length come back too
// (tb, ql, ps), so the caller need not read them again.
__device__ __forceinline__ void find_tile(const SeqLayout& sl, int g, int slot, int lane, int& fb,
                                          int& ft, int& tb, int& ql, int& ps,
                                          int rows = kPrefillRows) {
  __shared__ int s_member[2 * kGroupTiles];   // (request, tiles) of the group's requests
  fb = -1;
  ft = 0;
  tb = ql = ps = 0;
  // per-lane tiles and inclusive tile prefix of requests b0 + lane (the
  // first chunk is kept: batches of up to 64 requests are scanned once)
  auto scan = [&](int b0, int& nt, int& incl, int& cb, int& cq, int& cp) {
    const int bb = b0 + lane;
    cb = cq = cp = 0;
    if (bb < sl.batch) {
      cb = sl.cum[bb];
      cq = sl.cum[bb + 1] - cb;
      cp = sl.past[bb];
    }
    nt = cq >= 2 ? (cq * g + rows - 1) / rows : 0;
    incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
  };
  int nt0, incl0, cb0, cq0, cp0;
  scan(0, nt0, incl0, cb0, cq0, cp0);
  // pass 1: the request whose tiles hold `slot` in request order (its start
  // `mine_start`), and the total number of tiles
  int base = 0, mine_start = -1;
  for (int b0 = 0; b0 < sl.batch; b0 += 64) {
    int nt = nt0, incl = incl0, cb = cb0, cq = cq0, cp = cp0;
    if (b0 > 0) scan(b0, nt, incl, cb, cq, cp);
    const bool mine = nt > 0 && slot >= base + incl - nt && slot < base + incl;
    const unsigned long long bal = __ballot(mine);
    if (bal) mine_start = base + __shfl(incl - nt, __builtin_ctzll(bal), 64);
    base += __shfl(incl, 63, 64);
  }
  if (mine_start < 0) return;
  const int gt = base <= kGroupTiles ? 1 : kGroupTiles;   // tiles per group (at least)
  const int group = mine_start / gt;
  // pass 2: the group's requests (at most kGroupTiles: each starts at a
  // distinct slot of the group's range), in order, into s_member
  int members = 0, first = -1;
  base = 0;
  for (int b0 = 0; b0 < sl.batch; b0 += 64) {
    int nt = nt0, incl = incl0, cb = cb0, cq = cq0, cp = cp0;
    if (b0 > 0) scan(b0, nt, incl, cb, cq, cp);
    const int bb = b0 + lane;
    const int start = base + incl - nt;
    const bool in = nt > 0 && start / gt == group;
    const unsigned long long bal = __ballot(in);
    if (bal) {
      if (first < 0) first = __shfl(start, __builtin_ctzll(bal), 64);
      if (in) {
        const int m = members + __builtin_popcountll(bal & ((1ull << lane) - 1));
        s_member[2 * m] = bb;
        s_member[2 * m + 1] = nt;
      }
      members += __builtin_popcountll(bal);
    }
    base += __shfl(incl, 63, 64);
    if (base / gt > group) break;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the writes above are visible to the wave
  __builtin_amdgcn_wave_barrier();
  const int mb = lane < members ? s_member[2 * lane] : 0;
  const int mn = lane < members ? s_member[2 * lane + 1] : 0;
  // rank-major position: P(r) = sum over members of min(n, r) slots precede rank r
  const int k = slot - first;
  int r_lo = 0, r_hi = 0;
  {
    int mx = mn;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
    r_hi = mx;   // P(r_hi) = group size > k
  }
  while (r_hi - r_lo > 1) {   // invariant: P(r_lo) <= k < P(r_hi)
    const int mid = (r_lo + r_hi) >> 1;
    if (wave_sum(min(mn, mid)) <= k) r_lo = mid; else r_hi = mid;
  }
  const int idx = k - wave_sum(min(mn, r_lo));
  // the idx-th member (in order) that has a tile of rank r_lo
  unsigned long long bal = __ballot(lane < members && mn > r_lo);
  for (int i = 0; i < idx; ++i) bal &= bal - 1;
  const int src = __builtin_ctzll(bal);
  fb = __shfl(mb, src, 64);
  ft = __shfl(mn, src, 64) - 1 - r_lo;
  // the chosen request's token range and past: from the first chunk's
  // registers when it lies there, else read
  if (fb < 64) {
    tb = __shfl(cb0, fb, 64);
    ql = __shfl(cq0, fb, 64);
    ps = __shfl(cp0, fb, 64);
  } else {
    tb = sl.cum[fb];
    ql = sl.cum[fb + 1] - tb;
    ps = sl.past[fb];
  }
}
__device__ __forceinline__ void find_tile(const SeqLayout& sl, int g, int slot, int lane, int& fb,
                                          int& ft, int rows = kPrefillRows) {
  int tb, ql, ps;
  find_tile(sl, g, slot, lane, fb, ft, tb, ql, ps, rows);
}

// Key range [lo, hi) that tile `tile` (of `rows` rows) of a request (q_len,
// past) needs, and how it is cut into pieces of whole key tiles of `kt` keys
// for `chunks` workgroups.
struct TileKeys {
  int lo, hi;              // admitted keys of any row of the tile
  int all_begin, all_tiles;
  int per_piece, pieces;
};
__device__ __forceinline__ TileKeys tile_keys(int tile, int q_len, int past, int g, int window,
                                              int cap, int chunks, int piece_tiles,
                                              int rows = kPrefillRows, int kt = 64) {
  TileKeys k;
  const int j_first = (tile * rows) / g;
  const int j_last = min(q_len - 1, (tile * rows + rows - 1) / g);
  k.hi = min(past + j_last + 1, cap);
  k.lo = window > 0 ? max(0, past + j_first + 1 - window) : 0;
  k.all_begin = k.lo & ~(kt - 1);
  k.all_tiles = k.hi > k.all_begin ? (k.hi - k.all_begin + kt - 1) / kt : 0;
  // piece_tiles > 0: pieces of about piece_tiles 64-key tiles (short tiles
  // stay whole), at most `chunks`; else `chunks` equal pieces
  const int pt = piece_tiles * 64 / kt;
  const int want = piece_tiles > 0 ? (k.all_tiles + pt - 1) / pt : chunks;
  const int n = max(1, min(chunks, want));
  k.per_piece = (k.all_tiles + n - 1) / n;
  k.pieces = k.per_piece > 0 ? (k.all_tiles + k.per_piece - 1) / k.per_piece : 1;
  return k;
}

// max / sum of a value with the one 32 lanes away (one lane-swap instruction)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the same with the lane 16 away within each half of the wave
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace
}  // namespace pa
