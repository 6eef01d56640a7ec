// Row-per-wave block-sparse prefill: the fp32 path and the fallback for
// shapes the MFMA kernel does not take.
//
// Softmax attention of one query row over its visible keys (sinks, earlier
// gists, the causal window, unfolded chunks: UniGist summary, Approach;
// Simplified Sparse Attention via Gist Tokens, abstract), walking the row's
// non-empty stream-ordered key tiles.  A wave holds one query; each lane takes
// one key of a 64-key slice (logit in fp32, masked only in PARTIAL tiles),
// the slice updates a running max / sum (online softmax), and lanes then own
// head-dimension columns of the output while the slice's probabilities are
// broadcast.  Arithmetic is fp32 throughout; no down-conversion.
#include <math.h>

#include "gsa_internal.h"

namespace gsa {
namespace {

template <typename T> __device__ inline float ld(const T* p);
template <> __device__ inline float ld<float>(const float* p) { return *p; }
template <> __device__ inline float ld<unsigned short>(const unsigned short* p) { return bf16_to_f32(*p); }

template <typename TO> __device__ inline void st(TO* p, float v);
template <> __device__ inline void st<float>(float* p, float v) { *p = v; }
template <> __device__ inline void st<unsigned short>(unsigned short* p, float v) {
  *p = (unsigned short)(pack_bf16x2(v, 0.f) & 0xffffu);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) v = fmaxf(v, __shfl_xor(v, j));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) v += __shfl_xor(v, j);
  return v;
}

constexpr int kMaxD = 256;

template <typename T, typename TO>
__global__ __launch_bounds__(64) void k_prefill_rowwave(
    Lay l, int d, const T* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const T* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh, const T* __restrict__ v,
    int64_t vsb, int64_t vst, int64_t vsh, TO* __restrict__ o, int64_t osb, int64_t ost,
    int64_t osh, float* __restrict__ lse, int Hq, int Hkv, int q_begin, int q_len, int bm, int nqt,
    const int* __restrict__ sel, const int* __restrict__ selg, const int8_t* __restrict__ table,
    const int* __restrict__ tile_cnt, const int* __restrict__ tile_list, float scale, int tmode) {
  const int r = blockIdx.x, hq = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int G = Hq / Hkv, h = hq / G;
  const int i = q_begin + r;
  const int qt = r / bm;
  const int t = tmode == 1 ? 0 : (tmode == 2 ? b : b * Hkv + h);   // table per (b, KV head) | one | per b
  __shared__ float qs[kMaxD];
  __shared__ int ssel[64], sselg[64];
  for (int e = lane; e < d; e += 64) qs[e] = ld(q + b * qsb + r * qst + hq * qsh + e);
  const size_t srow = ((size_t)b * Hkv + h) * q_len + r;
  if (sel && lane < l.k) ssel[lane] = sel[srow * l.k + lane];
  if (selg && lane < l.k2) sselg[lane] = selg[srow * l.k2 + lane];
  __syncthreads();

  const T* kb = k + b * ksb + h * ksh;
  const T* vb = v + b * vsb + h * vsh;
  const size_t trow = (size_t)t * nqt + qt;
  const int cnt = tile_cnt[trow];
  const int* list = tile_list + trow * l.nkt;
  const int8_t* codes = table + trow * l.nkt;

  float m = kNegBig, lsum = 0.f;
  float acc[kMaxD / 64];
#pragma unroll
  for (int e = 0; e < kMaxD / 64; ++e) acc[e] = 0.f;

  for (int idx = 0; idx < cnt; ++idx) {
    const int kt = list[idx];
    const int code = codes[kt];
    int kind, u0, u1;
    tile_span(l, kt, kind, u0, u1);
    for (int c0 = u0; c0 < u1; c0 += 64) {
      const int u = c0 + lane;
      const bool inb = u < u1;
      const int p = inb ? pos_of(l, kind, u) : 0;
      const bool vis = inb && (code == 2 || key_visible(l, i, kind, u, p, ssel, sselg));
      float s = -__builtin_inff();
      if (vis) {
        const T* kr = kb + (int64_t)p * kst;
        float dot = 0.f;
        for (int e = 0; e < d; ++e) dot = fmaf(qs[e], ld(kr + e), dot);
        s = dot * scale;
      }
      const float mt = wave_max(s);
      const float mn = fmaxf(m, mt);
      const float alpha = expf(m - mn);
      const float pe = vis ? expf(s - mn) : 0.f;
      lsum = lsum * alpha + wave_sum(pe);
#pragma unroll
      for (int e = 0; e < kMaxD / 64; ++e) acc[e] *= alpha;
      m = mn;
      for (int j = 0; j < 64; ++j) {
        const float pj = __shfl(pe, j);
        if (pj == 0.f) continue;
        const int pos = __shfl(p, j);
        const T* vr = vb + (int64_t)pos * vst;
#pragma unroll
        for (int e = 0; e < kMaxD / 64; ++e) {
          const int col = lane + 64 * e;
          if (col < d) acc[e] = fmaf(pj, ld(vr + col), acc[e]);
        }
      }
    }
  }
  const float inv = 1.f / lsum;
  TO* orow = o + b * osb + r * ost + hq * osh;
#pragma unroll
  for (int e = 0; e < kMaxD / 64; ++e) {
    const int col = lane + 64 * e;
    if (col < d) st(orow + col, acc[e] * inv);
  }
  if (lse && lane == 0) lse[((size_t)b * Hq + hq) * q_len + r] = m + logf(lsum);
}

}  // namespace

// Launched by gsa_attn_prefill (prefill_mfma.hip) for f32 inputs and for bf16
// shapes the MFMA kernel does not cover.
gsa_status launch_prefill_rowwave(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k,
                                  const gsa_tensor& v, const gsa_tensor& o, float* lse, int B, int Hq,
                                  int Hkv, int q_begin, int q_len, int bm, int nqt, const int* sel,
                                  const int* selg, const int8_t* table, const int* tile_cnt,
                                  const int* tile_list, float scale, int tmode, hipStream_t st) {
  if (d > kMaxD) return fail(GSA_EUNSUPPORTED, "head dim %d > %d", d, kMaxD);
  dim3 grid(q_len, Hq, B);
#define GSA_ROWWAVE(T, TO)                                                                      \
  hipLaunchKernelGGL((k_prefill_rowwave<T, TO>), grid, dim3(64), 0, st, l, d, (const T*)q.ptr,   \
                     q.stride_b, q.stride_t, q.stride_h, (const T*)k.ptr, k.stride_b, k.stride_t, \
                     k.stride_h, (const T*)v.ptr, v.stride_b, v.stride_t, v.stride_h, (TO*)o.ptr, \
                     o.stride_b, o.stride_t, o.stride_h, lse, Hq, Hkv, q_begin, q_len, bm, nqt,   \
                     sel, selg, table, tile_cnt, tile_list, scale, tmode)
  if (q.dtype == GSA_F32) {
    if (o.dtype == GSA_F32) GSA_ROWWAVE(float, float);
    else GSA_ROWWAVE(float, unsigned short);
  } else {
    if (o.dtype == GSA_F32) GSA_ROWWAVE(unsigned short, float);
    else GSA_ROWWAVE(unsigned short, unsigned short);
  }
#undef GSA_ROWWAVE
  return launch_status("gsa_attn_prefill (row-wave)");
}

}  // namespace gsa
