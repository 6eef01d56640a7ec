// Wave-level selection networks shared by the selection kernels: a total
// order on (score, id) -- higher score first, then lower id (the tie rule of
// the selection: Simplified Sparse Attention via Gist Tokens, abstract, with
// ties to the lower chunk index) -- a 64-lane bitonic sort, the merge of two
// best-first lists, and the placement of the chosen ids in ascending order.
#pragma once

#include <limits.h>

#include "gsa_internal.h"

namespace gsa {

__device__ inline bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}
// The same order evaluated without short-circuit (no branches in unrolled
// per-lane loops).
__device__ inline bool better_nb(float s1, int i1, float s2, int i2) {
  return (bool)((unsigned)(s1 > s2) | ((unsigned)(s1 == s2) & (unsigned)(i1 < i2)));
}

// Value of lane ^ j for a constant j (the networks below unroll fully):
// DPP quad permutes for 1 and 2, a row rotation by 8 for 8 (a rotation by half
// a 16-lane row is the xor), a swizzle for 4, and the row / half swaps for 16
// and 32, instead of an LDS permute.  The swaps exchange the two rows (or
// halves) of their operands, so the partner's value is the second result in
// the lower row or half and the first in the upper.
__device__ inline int xor_lane(int v, int j) {
  const int lane = __lane_id();
  if (j == 1) return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if (j == 2) return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if (j == 8) return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  if (j == 4) return __builtin_amdgcn_ds_swizzle(v, 0x101F);                      // xor 4 in 32-lane groups
  if (j == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((lane & 16) ? sw[0] : sw[1]);
  }
  if (j == 32) {
    const auto sw = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return (int)((lane & 32) ? sw[0] : sw[1]);
  }
  return __shfl_xor(v, j);
}
__device__ inline float xor_lane(float v, int j) { return __int_as_float(xor_lane(__float_as_int(v), j)); }

// One compare-exchange stage of a 64-lane bitonic network: the lane keeps the
// better of (own, partner at lane ^ j) if keep_better, else the worse.
__device__ inline void cx(float& s, int& id, int j, bool keep_better) {
  const float os = xor_lane(s, j);
  const int oi = xor_lane(id, j);
  if (better(os, oi, s, id) == keep_better) {
    s = os;
    id = oi;
  }
}

// Sort 64 (score, id) pairs across the wave, best first.
__device__ inline void wave_sort_best_first(float& s, int& id) {
  const int lane = __lane_id();
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const bool up = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      cx(s, id, j, lower == up);
    }
  }
}

// Running best-first list (rs, ri) absorbs another best-first list (xs, xi).
__device__ inline void wave_merge(float& rs, int& ri, float xs, int xi) {
  const int lane = __lane_id();
  const float ys = __shfl(xs, 63 - lane);
  const int yi = __shfl(xi, 63 - lane);
  if (better(ys, yi, rs, ri)) {
    rs = ys;
    ri = yi;
  }
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) cx(rs, ri, j, (lane & j) == 0);
}

// Lanes [0, k) of a best-first list hold the chosen ids, INT_MAX where fewer
// than k were chosen; being the worst entries, those fill lanes [nv, k).
// Write the ids ascending into out[0, k), -1 padded: each lane counts the
// chosen ids smaller than its own, and equal ones in lower lanes, so no
// sorting network is needed and the ranks of the nv chosen lanes are always
// a permutation of [0, nv): every slot is written even if an id repeated.
// kept (if given, 64 entries) receives the same list, INT_MAX padded.
// Returns the number chosen.
__device__ inline int place_ascending(int v, int k, int* __restrict__ out, int* kept) {
  const int lane = __lane_id();
  const bool valid = lane < k && v != INT_MAX;
  const unsigned long long vmask = __ballot(valid);
  const int nv = __popcll(vmask);
  int rank = 0;
  for (int j = 0; j < k; ++j) {
    const int vj = __builtin_amdgcn_readlane(v, j);
    const bool vj_valid = (vmask >> j) & 1ull;
    rank += (vj_valid && (vj < v || (vj == v && j < lane))) ? 1 : 0;
  }
  if (valid) {
    out[rank] = v;   // rank < nv
    if (kept) kept[rank] = v;
  } else {
    if (lane < k) out[lane] = -1;   // lane >= nv
    if (kept) kept[lane] = INT_MAX;
  }
  return nv;
}


// A NaN score would break the total order the networks rely on; it ranks as
// -inf.  Tested on the bits: the build assumes no NaNs, so a float
// comparison would be folded away.
__device__ inline float nan_to_neg_inf(float s) {
  return ((__float_as_uint(s) & 0x7fffffffu) > 0x7f800000u) ? -__builtin_inff() : s;
}

}  // namespace gsa
