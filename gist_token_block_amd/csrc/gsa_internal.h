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

// Layout as the kernels see it (passed by value).
struct Lay {
  int S, c, g, P, W1, k;        // W1 = max(window, 1)
  int G2, g2, k2, P2, GP;       // G2 == 0: single level; GP = G2 * P
  int L;                        // key positions [0, L)
  int nstr;                     // streams in key order
  int kind[4], len[4], tile0[4], ntile[4];
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
    int f = y / l.P, r = y - f * l.P;
    if (kind == K_RAW) return f * l.c + imin(r, l.c);
    if (kind == K_GIST) return f * l.g + imax(0, r - l.c);
    return 0;
  }
  int f2 = y / l.P2, r2 = y - f2 * l.P2;
  if (kind == K_GIST2) return f2 * l.g2 + imax(0, r2 - l.GP);
  int rr = imin(r2, l.GP);
  int f = rr / l.P, r = rr - f * l.P;
  if (kind == K_RAW) return (f2 * l.G2 + f) * l.c + imin(r, l.c);
  return (f2 * l.G2 + f) * l.g + imax(0, r - l.c);
}

// Position of the u-th token of `kind`.
__host__ __device__ inline int pos_of(const Lay& l, int kind, int u) {
  if (kind == K_SINK) return u;
  if (l.G2 == 0) {
    if (kind == K_RAW) {
      int m = u / l.c;
      return l.S + m * l.P + (u - m * l.c);
    }
    int m = u / l.g;
    return l.S + m * l.P + l.c + (u - m * l.g);
  }
  if (kind == K_GIST2) {
    int gr = u / l.g2;
    return l.S + gr * l.P2 + l.GP + (u - gr * l.g2);
  }
  if (kind == K_RAW) {
    int m = u / l.c, r = u - m * l.c, gr = m / l.G2, j = m - gr * l.G2;
    return l.S + gr * l.P2 + j * l.P + r;
  }
  int m = u / l.g, t = u - m * l.g, gr = m / l.G2, j = m - gr * l.G2;
  return l.S + gr * l.P2 + j * l.P + l.c + t;
}

// Key tile -> (stream kind, first and one-past-last stream index).
__host__ __device__ inline void tile_span(const Lay& l, int kt, int& kind, int& u0, int& u1) {
  int s = 0;
  while (s + 1 < l.nstr && kt >= l.tile0[s + 1]) ++s;
  kind = l.kind[s];
  u0 = (kt - l.tile0[s]) * l.bn;
  u1 = imin(u0 + l.bn, l.len[s]);
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
    int gr = (u / l.g) / l.G2;
    for (int e = 0; e < l.k2; ++e)
      if (selg[e] == gr) return true;
    return false;
  }
  int m = u / l.c;
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

// Round-to-nearest-even fp32 -> bf16 pair packed in one dword (lo = a).
__device__ inline unsigned pack_bf16x2(float a, float b) {
  unsigned ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua = (ua + 0x7fffu + ((ua >> 16) & 1u)) >> 16;
  ub = (ub + 0x7fffu + ((ub >> 16) & 1u)) & 0xffff0000u;
  return ua | ub;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;   // finite "minus infinity" for running maxima

}  // namespace gsa
