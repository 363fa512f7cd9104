// Prefill / chunked-prefill attention over the paged pool with fp16 MFMA.
//
// Online-softmax tiled attention (GroupQueryAttention CPU Implementation
// Notes, "Flash Attention Path": QK on a KV block, causal + local-window
// masking, running max/sum with exp(m_old - m_new) rescale, fused SV
// accumulate, 1/l at the end) with softcap applied to the scaled score before
// masking (PagedAttention -- CUDA Design Document, section 8.5 note) and the
// window of W positions ending at the query (section 4.5).  Tiles address the
// pool one key row at a time through block_table, so a tile may straddle pages
// of any power-of-two block size (the straddling limit of section 18.1 does
// not arise).
//
// One workgroup = 4 waves = 128 query rows of one kv head; a row is a (query
// token, head-in-group) pair, token-major, so every K/V tile staged in LDS is
// shared by all G heads of the group.  Each wave owns 32 rows and computes
//   S^T[key][row] = K[key][:] . Q[row][:]          (v_mfma_f32_32x32x16_f16)
// so that the score accumulator already has the B-operand layout of the PV
// product O^T[d][row] += V^T[d][key] P^T[key][row]: the probabilities go from
// registers to the MFMA without an LDS round trip.  V is stored transposed in
// LDS (with the key order of the accumulator layout: bits 2 and 3 of the key
// index swapped inside each 16-key group) so that both MFMA operands are plain
// 16-byte LDS reads.  Scores are in log2 units; the row max is shared by the
// two lanes holding a row with one cross-lane swap per tile.
#include "pa_device.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int swap23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs a) {
  constexpr int ROWS = kPrefillRows;  // 128 rows = 4 waves x 32
  constexpr int KT = 64;              // keys per tile
  constexpr int KS = D / 16;          // MFMA k-steps over the head dim
  constexpr int DB = D / 32;          // 32-channel output blocks
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int KLD = D + 8;          // LDS row stride of K (halves)
  constexpr int VLD = KT + 8;         // LDS row stride of V^T (halves)

  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VLD];
  __shared__ uint8_t key_ok[KT];
  __shared__ int sh_b, sh_tile, sh_ntiles, sh_hole;

  const SeqLayout& sl = a.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int kvh = blockIdx.y;
  const int g = a.group;
  const int64_t HD = (int64_t)a.num_heads * D;

  if ((int)blockIdx.x == a.tiles) {
    // tokens owned by no request get zero rows (this kv head's columns)
    const int t0 = max(sl.cum[sl.batch], 0);
    const int width = g * CH;
    for (int64_t i = tid; i < (int64_t)(sl.tokens - min(t0, sl.tokens)) * width; i += 256) {
      const int t = t0 + (int)(i / width);
      const int cc = (int)(i % width);
      store16(a.out + t * HD + (int64_t)kvh * g * D + 8 * cc, u32x4{0, 0, 0, 0});
    }
    return;
  }

  // Map this workgroup to (request, tile) over requests with q_len >= 2.
  if (wave == 0) {
    const int slot = blockIdx.x;
    int base = 0, fb = -1, ft = 0, fn = 0;
    for (int b0 = 0; b0 < sl.batch; b0 += 64) {
      const int bb = b0 + lane;
      int nt = 0;
      if (bb < sl.batch) {
        const int ql = sl.cum[bb + 1] - sl.cum[bb];
        if (ql >= 2) nt = (ql * g + ROWS - 1) / ROWS;
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
        ft = slot - (base + __shfl(incl - nt, src, 64));
        fn = __shfl(nt, src, 64);
        break;
      }
      base += total;
    }
    if (lane == 0) {
      sh_b = fb;
      sh_tile = fn - 1 - ft;   // later (longer) tiles of a request are dispatched first
      sh_ntiles = fn;
    }
  }
  __syncthreads();
  const int b = sh_b;
  if (b < 0) return;
  const int tile = sh_tile;

  const int t_begin = sl.cum[b];
  const int q_len = sl.cum[b + 1] - t_begin;
  const int past = sl.past[b];
  const int cap = sl.maxblk << sl.block_shift;
  const int shift = sl.block_shift;
  const int bmask = (1 << shift) - 1;
  const int32_t* bt = sl.block_table + (int64_t)b * sl.maxblk;
  const int64_t tok_stride = (int64_t)a.kv_heads * D;
  const uint16_t* kbase = a.key_cache + (int64_t)kvh * D;
  const uint16_t* vbase = a.value_cache + (int64_t)kvh * D;

  // this lane's query row
  const int R = tile * ROWS + wave * 32 + l32;
  const int j = R / g;
  const int hh = R - j * g;
  const bool row_ok = j < q_len && t_begin + j < sl.tokens;
  const int pos = row_ok ? past + j : -1;
  const int t = t_begin + j;
  const int head = kvh * g + hh;

  // key range of the whole tile
  const int j_first = (tile * ROWS) / g;
  const int j_last = min(q_len - 1, (tile * ROWS + ROWS - 1) / g);
  const int hi = min(past + j_last + 1, cap);
  const int lo = a.window > 0 ? max(0, past + j_first + 1 - a.window) : 0;
  // range of this wave's rows (for the unmasked-tile fast path)
  const int wj0 = min((tile * ROWS + wave * 32) / g, q_len - 1);
  const int wj1 = min((tile * ROWS + wave * 32 + 31) / g, q_len - 1);
  const int wpos_min = past + wj0;
  const int wpos_max = past + wj1;

  // Q fragments (B operand): row l32, channels 16*ks + 8*hf .. +7
  h8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (row_ok) {
      const uint16_t* qrow = a.query + (int64_t)t * HD + (int64_t)head * D;
      const int c = 2 * ks + hf;
      v = load16(qrow + 8 * c);
      if (a.rotary_dim > 0 && 8 * c < a.rotary_dim) {
        float rr[8];
        rotate_chunk(qrow, v, c, pos, a.cos, a.sin, a.rotary_dim, a.rotary_interleaved,
                     a.rotary_rows, rr);
        v = pack8(rr);
      }
    }
    qf[ks] = as_h8(v);
  }

  f16v acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = kNegInf, lsum = 0.f;
  const bool softcap = a.use_softcap != 0;

  for (int kt0 = lo & ~(KT - 1); kt0 < hi; kt0 += KT) {
    __syncthreads();
    if (tid == 0) sh_hole = 0;
    __syncthreads();
    // ---- stage K tile [KT][D] ----
    for (int i = tid; i < KT * CH; i += 256) {
      const int kk = i / CH;
      const int cc = i - kk * CH;
      const int tau = kt0 + kk;
      u32x4 v = u32x4{0, 0, 0, 0};
      bool ok = false;
      if (tau >= lo && tau < hi) {
        const int blk = bt[tau >> shift];
        if (blk >= 0 && blk < sl.num_blocks) {
          v = load16(kbase + ((int64_t)blk * (bmask + 1) + (tau & bmask)) * tok_stride + 8 * cc);
          ok = true;
        } else if (cc == 0) {
          sh_hole = 1;
        }
      }
      if (cc == 0) key_ok[kk] = ok;
      store16(&Ks[kk * KLD + 8 * cc], v);
    }
    // ---- stage V^T tile [D][KT] (groups of 4 keys, transposed in registers) ----
    for (int i = tid; i < (KT / 4) * CH; i += 256) {
      const int kg = i / CH;
      const int cc = i - kg * CH;
      const int kk0 = 4 * kg;
      uint16_t vv[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tau = kt0 + kk0 + r;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (tau >= lo && tau < hi) {
          const int blk = bt[tau >> shift];
          if (blk >= 0 && blk < sl.num_blocks)
            v = load16(vbase + ((int64_t)blk * (bmask + 1) + (tau & bmask)) * tok_stride + 8 * cc);
        }
        __builtin_memcpy(vv[r], &v, 16);
      }
      const int p0 = swap23(kk0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = (uint32_t)vv[0][e] | ((uint32_t)vv[1][e] << 16);
        w.y = (uint32_t)vv[2][e] | ((uint32_t)vv[3][e] << 16);
        *reinterpret_cast<uint2*>(&Vt[(8 * cc + e) * VLD + p0]) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K . Q^T for two 32-key blocks ----
    f16v s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const h8 ka = *reinterpret_cast<const h8*>(&Ks[(kb * 32 + l32) * KLD + 16 * ks + 8 * hf]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[ks], s[kb], 0, 0, 0);
      }
    }

    // ---- scale / softcap / mask (log2 units) ----
    const bool full = sh_hole == 0 && kt0 + KT - 1 <= wpos_min &&
                      (a.window <= 0 || kt0 >= wpos_max - a.window + 1) && kt0 + KT <= hi &&
                      kt0 >= lo;
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r];
        x = softcap ? tanh_fast(x * a.cap_in) * a.cap_out : x * a.score_scale;
        if (!full) {
          const int kk = kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const int tau = kt0 + kk;
          bool adm = tau <= pos && key_ok[kk];
          if (a.window > 0) adm = adm && tau >= pos - a.window + 1;
          x = adm ? x : kNegInf;
        }
        s[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float mu = mn == kNegInf ? 0.f : mn;
    const float alpha = exp2_fast(m - mu);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    // ---- P (fp16) as B operand; O^T += V^T . P^T ----
    h8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(s[kb][r] - mu);
        lsum += p;
        pf[2 * kb + (r >> 3)][r & 7] = (_Float16)p;
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const h8 va = *reinterpret_cast<const h8*>(&Vt[(db * 32 + l32) * VLD + 16 * ks + 8 * hf]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[ks], acc[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store ----
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (row_ok) {
    uint16_t* orow = a.out + (int64_t)t * HD + (int64_t)head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int head_size, dim3 grid, hipStream_t st) {
  switch (head_size) {
    case 64: hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL(prefill_kernel<256>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
