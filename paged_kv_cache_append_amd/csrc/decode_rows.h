// Decode rows: the query token a row of the split-KV decode stands for and
// the split layout of its admitted key interval.  Shared by the plan, merge
// and decode kernels (decode.hip) and the latent-attention kernel (mla.hip),
// which must all agree on it.
#pragma once

#include "pa_device.h"

namespace pa {
namespace {

struct RowInfo {
  int t, b, pos, lo, hi, nsplit;
};

// Resolve the query token a decode row stands for and the split layout of its
// admitted key interval [lo, hi).  Identical in the plan, decode and merge
// kernels.  Returns false when the row has no work for the decode kernel.
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

}  // namespace
}  // namespace pa
