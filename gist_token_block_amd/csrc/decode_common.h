// Pieces shared by the decode kernels: the 64-row block configuration, the
// LDS swizzles of staged K and V rows, device-scope loads and stores of split
// partials, and visible-row segments.
#pragma once

#include "gsa_internal.h"

namespace gsa {
namespace dec {

constexpr int kThreads = 256;
constexpr int kRows = 64;          // rows per staged block (double buffered)
constexpr int kMaxSeg = 3 + 64 + 64;
constexpr int kMaxSplit = 64;      // most splits per (batch, KV head)

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* glb_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

template <int D> struct DCfg {
  static constexpr int PPR = D / 8;          // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;       // rows per 1 KB wave load
  static constexpr int NIW = kRows / RPI / 4;  // wave loads per block per wave
  static constexpr int KS = D / 32;          // k-steps of the QK product (K = 32)
  static constexpr int MT = D / 16;          // 16-row tiles of O^T
};
// Row r keeps its 16-byte piece p at slot p ^ swz(r) (see the prefill kernel).
template <int D> __device__ inline int dswz_k(int r) { return r & (D / 8 - 1); }
template <int D> __device__ inline int dswz_v(int r) { return (4 * (r & 3)) & (D / 8 - 1); }

__device__ inline void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Visible-row segments of one (batch, KV head).
struct Segs {
  int n;
  int start[kMaxSeg + 1];  // first virtual row of each segment; start[n] = total
  int base[kMaxSeg];       // first position (contiguous) or first stream index
  int kind[kMaxSeg];       // -1: contiguous positions; else stream kind
};

__device__ inline int seg_pos(const Lay& l, const Segs& s, int v) {
  int lo = 0, hi = s.n - 1;            // last segment with start <= v
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.start[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  const int off = v - s.start[lo];
  return s.kind[lo] < 0 ? s.base[lo] + off : pos_of(l, s.kind[lo], s.base[lo] + off);
}

// A split partial per (batch, KV head, slot, query head): O (D floats), then
// the running max in log2 units, the sum of the bf16 P that O is built from,
// and the sum of the unrounded P (which gives the log-sum-exp).
constexpr int kPartExtra = 3;

}  // namespace dec
}  // namespace gsa
