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
// `rows` rows (token x head-in-group) each; later (longer) tiles of a request
// come first.  b = -1 past the last tile.  Called by a whole wave; the results
// are the same in every lane.
__device__ __forceinline__ void find_tile(const SeqLayout& sl, int g, int slot, int lane, int& fb,
                                          int& ft, int rows = kPrefillRows) {
  int base = 0;
  fb = -1;
  ft = 0;
  for (int b0 = 0; b0 < sl.batch; b0 += 64) {
    const int bb = b0 + lane;
    int nt = 0;
    if (bb < sl.batch) {
      const int ql = sl.cum[bb + 1] - sl.cum[bb];
      if (ql >= 2) nt = (ql * g + rows - 1) / rows;
    }
    int incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, 63, 64);
    if (slot < base + total) {
      const bool mine = nt > 0 && slot >= base + incl - nt && slot < base + incl;
      const unsigned long long bal = __ballot(mine);
      const int src = __builtin_ctzll(bal);
      fb = b0 + src;
      const int fn = __shfl(nt, src, 64);
      ft = fn - 1 - (slot - (base + __shfl(incl - nt, src, 64)));
      return;
    }
    base += total;
  }
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
