// Internal declarations shared by the libgsa HIP sources (gfx950 only).
//
// Layout arithmetic.  The interleaved sequence is n_sink sinks, then chunks of
// c raw tokens each followed by g gists (Study page "A Silver Bullet or a
// Compromise for Full Attention?", §2; UniGist summary, Approach); with two
// levels a group is G2 chunks followed by g2 level-2 gists (Forget, Then
// Recall ... Gist Sparse Attention, abstract).  Every token kind forms a
// "stream" ordered by position; the kernels address keys as (stream, index)
// and convert to positions with the closed forms below.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include <string>

#include "gsa.h"

namespace gsa {

enum Kind : int { K_SINK = 0, K_GIST2 = 1, K_GIST = 2, K_RAW = 3 };

// Division by a divisor fixed at launch: q = (mulhi(m, n) + n) >> s with
// s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1 (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  Exact for 0 <= n < 2^31, which covers every index
// here (positions and stream indices are int).
struct FDiv {
  unsigned m, s;
};

inline FDiv make_fdiv(unsigned d) {
  unsigned s = 0;
  while ((1ull << s) < d) ++s;
  const unsigned long long m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FDiv{(unsigned)m, s};
}

__host__ __device__ inline int fdiv(const FDiv& f, int n) {
  const unsigned un = (unsigned)n;
  const unsigned t = (unsigned)(((unsigned long long)f.m * un) >> 32);
  return (int)((t + un) >> f.s);
}

// Stream index -> position without branches: with m = u / per, r = u % per,
// grp = m / G, j = m % G: pos = base + grp * stride2 + j * stride1 + r.
// Single-level streams use G = 2^30 (grp = 0).
struct StreamMap {
  FDiv dper, dG;
  int per, G, stride1, stride2, base;
};

__host__ __device__ inline int map_pos(const StreamMap& sm, int u) {
  const int m = fdiv(sm.dper, u), r = u - m * sm.per;
  const int grp = fdiv(sm.dG, m), j = m - grp * sm.G;
  return sm.base + grp * sm.stride2 + j * sm.stride1 + r;
}

// Layout as the kernels see it (passed by value).
struct Lay {
  int S, c, g, P, W1, k;        // W1 = max(window, 1)
  int G2, g2, k2, P2, GP;       // G2 == 0: single level; GP = G2 * P
  int L;                        // key positions [0, L)
  FDiv dc, dg, dP, dG2, dg2, dP2;
  int nstr;                     // streams in key order
  int kind[4], len[4], tile0[4];
  StreamMap smap[4];            // per stream slot
  int bn, nkt;                  // key tile width and count
};

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ inline int iclamp(int x, int lo, int hi) { return imin(imax(x, lo), hi); }
// length of [a0,a1) ∩ [b0,b1)
__host__ __device__ inline int overlap(int a0, int a1, int b0, int b1) {
  return imax(0, imin(a1, b1) - imax(a0, b0));
}

// Tokens of `kind` at positions < x.
__host__ __device__ inline int count_below(const Lay& l, int kind, int x) {
  if (x <= 0) return 0;
  if (kind == K_SINK) return imin(x, l.S);
  int y = x - l.S;
  if (y <= 0) return 0;
  if (l.G2 == 0) {
    int f = fdiv(l.dP, y), r = y - f * l.P;
    if (kind == K_RAW) return f * l.c + imin(r, l.c);
    if (kind == K_GIST) return f * l.g + imax(0, r - l.c);
    return 0;
  }
  int f2 = fdiv(l.dP2, y), r2 = y - f2 * l.P2;
  if (kind == K_GIST2) return f2 * l.g2 + imax(0, r2 - l.GP);
  int rr = imin(r2, l.GP);
  int f = fdiv(l.dP, rr), r = rr - f * l.P;
  if (kind == K_RAW) return (f2 * l.G2 + f) * l.c + imin(r, l.c);
  return (f2 * l.G2 + f) * l.g + imax(0, r - l.c);
}

// Position of the u-th token of `kind`.
__host__ __device__ inline int pos_of(const Lay& l, int kind, int u) {
  if (kind == K_SINK) return u;
  if (l.G2 == 0) {
    if (kind == K_RAW) {
      int m = fdiv(l.dc, u);
      return l.S + m * l.P + (u - m * l.c);
    }
    int m = fdiv(l.dg, u);
    return l.S + m * l.P + l.c + (u - m * l.g);
  }
  if (kind == K_GIST2) {
    int gr = fdiv(l.dg2, u);
    return l.S + gr * l.P2 + l.GP + (u - gr * l.g2);
  }
  if (kind == K_RAW) {
    int m = fdiv(l.dc, u), r = u - m * l.c, gr = fdiv(l.dG2, m), j = m - gr * l.G2;
    return l.S + gr * l.P2 + j * l.P + r;
  }
  int m = fdiv(l.dg, u), t = u - m * l.g, gr = fdiv(l.dG2, m), j = m - gr * l.G2;
  return l.S + gr * l.P2 + j * l.P + l.c + t;
}

// Level-1 chunk of the u-th raw token / group of the u-th level-1 gist.
__host__ __device__ inline int raw_chunk(const Lay& l, int u) { return fdiv(l.dc, u); }
__host__ __device__ inline int gist_group(const Lay& l, int u) { return fdiv(l.dG2, fdiv(l.dg, u)); }

// Key tile -> (stream slot, stream kind, first and one-past-last stream index).
__host__ __device__ inline int tile_span(const Lay& l, int kt, int& kind, int& u0, int& u1) {
  // straight-line: unused slots have tile0 = nkt, so they never match
  const int s = (kt >= l.tile0[1]) + (kt >= l.tile0[2]) + (l.nstr > 3 && kt >= l.tile0[3]);
  const int t0 = s == 0 ? l.tile0[0] : s == 1 ? l.tile0[1] : s == 2 ? l.tile0[2] : l.tile0[3];
  const int ln = s == 0 ? l.len[0] : s == 1 ? l.len[1] : s == 2 ? l.len[2] : l.len[3];
  kind = s == 0 ? l.kind[0] : s == 1 ? l.kind[1] : s == 2 ? l.kind[2] : l.kind[3];
  u0 = (kt - t0) * l.bn;
  u1 = imin(u0 + l.bn, ln);
  return s;
}

__host__ __device__ inline StreamMap slot_map(const Lay& l, int s) {
  return s == 0 ? l.smap[0] : s == 1 ? l.smap[1] : s == 2 ? l.smap[2] : l.smap[3];
}

// Is key (kind, stream index u, position p) visible to the query at i?
// sel: the query's chosen chunks (k entries, -1 padded); selg: chosen groups.
__device__ inline bool key_visible(const Lay& l, int i, int kind, int u, int p,
                                   const int* sel, const int* selg) {
  if (p > i) return false;
  if (kind == K_SINK || kind == K_GIST2) return true;
  if (kind == K_GIST && l.G2 == 0) return true;
  if (i - p < l.W1) return true;
  if (kind == K_GIST) {
    int gr = gist_group(l, u);
    for (int e = 0; e < l.k2; ++e)
      if (selg[e] == gr) return true;
    return false;
  }
  int m = raw_chunk(l, u);
  for (int e = 0; e < l.k; ++e)
    if (sel[e] == m) return true;
  return false;
}

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
gsa_status fail(gsa_status st, const char* fmt, ...);
// Fill `out` from the public layout for a sequence of L positions and key
// tiles of width bn.  Returns GSA_OK or GSA_EINVAL (message set).
gsa_status make_lay(const gsa_layout* layout, int L, int bn, Lay* out);
gsa_status check_tensor(const char* name, const gsa_tensor& t, int d, bool need_bf16_or_f32 = true);
gsa_status launch_status(const char* what);

// ---------------------------------------------------------------- device utilities
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16_to_f32(unsigned short h) { return __uint_as_float(((unsigned)h) << 16); }
__device__ inline float lo_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 pair packed in one dword (lo = a);
// a single v_cvt_pk_bf16_f32 on gfx950.
__device__ inline unsigned pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(unsigned, h);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

}  // namespace gsa
