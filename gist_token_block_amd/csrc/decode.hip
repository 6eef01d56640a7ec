// Split-K decode (gsa_attn_decode): one query token per sequence attends to
// the sinks, every gist (two levels: every level-2 gist and the level-1 gists
// of the kept groups), its causal window and the raw tokens of its unfolded
// chunks (Simplified Sparse Attention via Gist Tokens, abstract; Forget, Then
// Recall ... Gist Sparse Attention, abstract; UniGist summary, Approach).
//
// The visible rows of one (batch, KV head) are enumerated as disjoint
// segments -- sinks before the window, gists before the window, the kept
// groups' level-1 gists before the window, the window itself, each unfolded
// chunk's raws before the window -- so every row is read exactly once.  The
// rows are cut into splits of 128; one workgroup (4 waves) per (split, KV
// head, batch) stages 64 rows of K and V at a time to LDS with 16-byte loads
// (a chunk's raws are contiguous in the [B, Hkv, kv_len, d] cache), and each
// wave takes 16 of them for all G query heads of the KV group at once:
//   S^T (16 keys x 16 head slots) = K q^T   v_mfma_f32_16x16x32_bf16
//   O^T (16 d x 16 head slots)   += V^T P^T v_mfma_f32_16x16x16_bf16
// The S accumulator layout (lane = head slot, 4 keys) is exactly the B operand
// layout of the 16x16x16 product, so P never leaves registers.  Waves keep
// separate (max, sum, O) partials; they are merged in LDS, written to the
// workspace, and a second kernel merges the splits (log-sum-exp weights).
#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;          // rows staged per step
constexpr int kRowsPerSplit = 128;
constexpr int kMaxSeg = 3 + 64 + 64;

template <int D> struct DCfg {
  static constexpr int KP = D + 8;
  static constexpr int VP = D + 8;
  static constexpr int PPR = D / 8;
  static constexpr int KS = D / 32;   // k-steps of the QK product (K = 32)
  static constexpr int MT = D / 16;   // 16-row tiles of O^T
};

// Visible-row segments of one (batch, KV head).
struct Segs {
  int n;
  int start[kMaxSeg + 1];  // first virtual row of each segment; start[n] = total
  int base[kMaxSeg];       // first position (contiguous) or first stream index
  int kind[kMaxSeg];       // -1: contiguous positions; else stream kind
};

__device__ inline int seg_pos(const Lay& l, const Segs& s, int v) {
  int j = 0;
  while (j + 1 < s.n && s.start[j + 1] <= v) ++j;
  const int off = v - s.start[j];
  return s.kind[j] < 0 ? s.base[j] + off : pos_of(l, s.kind[j], s.base[j] + off);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_decode_split(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qsh,
    const unsigned short* __restrict__ kc, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ vc, int64_t vsb, int64_t vst, int64_t vsh, int Hq, int Hkv,
    int kv_len, const int* __restrict__ sel, const int* __restrict__ selg, float c2,
    float* __restrict__ ws, int nsplit) {
  using C = DCfg<D>;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int G = Hq / Hkv;
  const int i = kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);

  __shared__ Segs segs;
  __shared__ __attribute__((aligned(16))) unsigned short stage[kRows * (C::KP + C::VP)];
  unsigned short* Klds = stage;
  unsigned short* Vlds = stage + kRows * C::KP;

  if (tid == 0) {
    int n = 0, tot = 0;
    auto add = [&](int kind, int base, int len) {
      if (len <= 0) return;
      segs.start[n] = tot;
      segs.base[n] = base;
      segs.kind[n] = kind;
      tot += len;
      ++n;
    };
    add(-1, 0, imin(l.S, lo));
    const size_t srow = (size_t)b * Hkv + h;
    if (l.G2 == 0) {
      add(K_GIST, 0, count_below(l, K_GIST, lo));
    } else {
      add(K_GIST2, 0, count_below(l, K_GIST2, lo));
      const int gl = count_below(l, K_GIST, lo), per = l.G2 * l.g;
      const int ngr = count_below(l, K_GIST2, i) / l.g2;   // groups complete before i
      for (int e = 0; e < l.k2; ++e) {
        const int gr = selg[srow * l.k2 + e];
        if (gr >= 0 && gr < ngr) add(K_GIST, gr * per, iclamp(gl - gr * per, 0, per));
      }
    }
    add(-1, lo, i - lo + 1);
    const int nch = count_below(l, K_GIST, i) / l.g;          // chunks complete before i
    for (int e = 0; e < l.k; ++e) {
      const int m = sel[srow * l.k + e];
      if (m < 0 || m >= nch) continue;   // ids outside the candidates are ignored
      const int st = pos_of(l, K_RAW, m * l.c);
      add(-1, st, iclamp(lo - st, 0, l.c));
    }
    segs.start[n] = tot;
    segs.n = n;
  }

  // q^T operands: lane = head slot `col` (valid if < G), d = 8 grp + 32 ks
  bf16x8 qreg[C::KS];
  {
    const unsigned short* qrow = q + b * qsb + (int64_t)(h * G + imin(col, G - 1)) * qsh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * grp + 32 * ks);
      if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __syncthreads();

  const int total = segs.start[segs.n];
  const int v_begin = split * kRowsPerSplit;
  const int v_end = imin(v_begin + kRowsPerSplit, total);
  const unsigned short* kb = kc + b * ksb + h * ksh;
  const unsigned short* vb = vc + b * vsb + h * vsh;

  f32x4 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;

  for (int vb0 = v_begin; vb0 < v_end; vb0 += kRows) {
    constexpr int RPP = kThreads / C::PPR;
#pragma unroll
    for (int it = 0; it < kRows / RPP; ++it) {
      const int rr = tid / C::PPR + RPP * it;
      const int piece = tid % C::PPR;
      const int vv = vb0 + rr;
      u32x4 wk = u32x4{0u, 0u, 0u, 0u}, wv = wk;
      if (vv < v_end) {
        const int p = seg_pos(l, segs, vv);
        wk = *reinterpret_cast<const u32x4*>(kb + (int64_t)p * kst + piece * 8);
        wv = *reinterpret_cast<const u32x4*>(vb + (int64_t)p * vst + piece * 8);
      }
      *reinterpret_cast<u32x4*>(&Klds[rr * C::KP + piece * 8]) = wk;
      *reinterpret_cast<u32x4*>(&Vlds[rr * C::VP + piece * 8]) = wv;
    }
    __syncthreads();

    const int r0 = 16 * wave;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Klds[(r0 + col) * C::KP + 8 * grp + 32 * ks]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], s, 0, 0, 0);
    }
    // s[e]: key row r0 + 4 grp + e, head slot col
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (vb0 + r0 + 4 * grp + e >= v_end) s[e] = -__builtin_inff();
      mx = fmaxf(mx, s[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -m_new));
      ps += s[e];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const u32x2 pw = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    const bf16x4 pb = __builtin_bit_cast(bf16x4, pw);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      oacc[mt] *= alpha;
      const int dcol = 16 * mt + col;
      const unsigned short* vr = &Vlds[(r0 + 4 * grp) * C::VP + dcol];
      const unsigned w0 = (unsigned)vr[0] | ((unsigned)vr[C::VP] << 16);
      const unsigned w1 = (unsigned)vr[2 * C::VP] | ((unsigned)vr[3 * C::VP] << 16);
      const bf16x4 a = __builtin_bit_cast(bf16x4, u32x2{w0, w1});
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, oacc[mt], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- merge the 4 waves' partials (reuse the K/V staging memory)
  float* cm = reinterpret_cast<float*>(stage);         // [4][16]
  float* cl = cm + 4 * 16;                             // [4][16]
  float* co = cl + 4 * 16;                             // [4][16][D]
  static_assert(kRows * (DCfg<D>::KP + DCfg<D>::VP) * 2 >= (128 + 64 * D) * 4, "LDS reuse too small");
  if (grp == 0) {
    cm[wave * 16 + col] = m_run;
    cl[wave * 16 + col] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) co[(wave * 16 + col) * D + 16 * mt + 4 * grp + e] = oacc[mt][e];
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int hd = x / D, dd = x - hd * D;
    float M = kNegBig;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w * 16 + hd]);
    float L = 0.f, O = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(cm[w * 16 + hd] - M);
      L += cl[w * 16 + hd] * f;
      O += co[(w * 16 + hd) * D + dd] * f;
    }
    float* part = ws + ((((size_t)b * Hkv + h) * nsplit + split) * G + hd) * (D + 2);
    part[dd] = O;
    if (dd == 0) {
      part[D] = M;
      part[D + 1] = L;
    }
  }
}

template <int D, typename TO>
__global__ __launch_bounds__(D) void k_decode_combine(const float* __restrict__ ws, int Hq, int Hkv,
                                                      int nsplit, TO* __restrict__ o, int64_t osb,
                                                      int64_t osh, float* __restrict__ lse) {
  const int hq = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
  const int G = Hq / Hkv, h = hq / G, hd = hq - h * G;
  const float* base = ws + (((size_t)b * Hkv + h) * nsplit * G + hd) * (D + 2);
  const size_t step = (size_t)G * (D + 2);
  float M = kNegBig;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[s * step + D]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = __builtin_amdgcn_exp2f(base[s * step + D] - M);
    L += base[s * step + D + 1] * f;
    O += base[s * step + dd] * f;
  }
  const float val = O / L;
  TO* orow = o + b * osb + hq * osh;
  if constexpr (sizeof(TO) == 4) {
    orow[dd] = val;
  } else {
    orow[dd] = (TO)(pack_bf16x2(val, 0.f) & 0xffffu);
  }
  if (lse && dd == 0) lse[(size_t)b * Hq + hq] = (M + __log2f(L)) * kLn2;
}

// Upper bound of the visible rows of one decode query.
int row_bound(const Lay& l, int kv_len) {
  const int i = kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);
  long long n = imin(l.S, lo) + (i - lo + 1) + (long long)l.k * l.c;
  if (l.G2 == 0) n += count_below(l, K_GIST, lo);
  else n += count_below(l, K_GIST2, lo) + (long long)l.k2 * l.G2 * l.g;
  return (int)n;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" size_t gsa_decode_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                             int32_t d, int32_t kv_len) {
  Lay l;
  if (make_lay(layout, kv_len, 64, &l) != GSA_OK || kv_len < 1 || Hkv < 1 || Hq % Hkv) return 0;
  const int ns = (row_bound(l, kv_len) + kRowsPerSplit - 1) / kRowsPerSplit;
  return (size_t)B * Hkv * ns * (Hq / Hkv) * (d + 2) * sizeof(float);
}

extern "C" gsa_status gsa_attn_decode(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                                      gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B, int32_t Hq,
                                      int32_t Hkv, int32_t d, int32_t kv_len, const int32_t* sel,
                                      const int32_t* sel_groups, float scale, void* ws, size_t ws_bytes,
                                      void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, kv_len, 64, &l);
  if (st != GSA_OK) return st;
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("o", o, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k_cache.dtype != GSA_BF16 || v_cache.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "decode takes bf16 q and caches");
  if (o.dtype != GSA_F32 && o.dtype != GSA_BF16) return fail(GSA_EINVAL, "o dtype");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (Hq / Hkv > 16) return fail(GSA_EUNSUPPORTED, "more than 16 query heads per KV head");
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (kv_len < 1) return fail(GSA_EINVAL, "kv_len %d < 1", kv_len);
  if (l.k > 64 || l.k2 > 64) return fail(GSA_EUNSUPPORTED, "top_k and l2_top_k are limited to 64");
  if (l.k > 0 && !sel) return fail(GSA_EINVAL, "sel is required when top_k > 0");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is required with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  const size_t need = gsa_decode_workspace_bytes(layout, B, Hq, Hkv, d, kv_len);
  if (!ws || ws_bytes < need) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  const int ns = (row_bound(l, kv_len) + kRowsPerSplit - 1) / kRowsPerSplit;
  hipStream_t s = (hipStream_t)stream;
  const float c2 = scale * kLog2e;
  float* w = (float*)ws;
#define GSA_SPLIT(D)                                                                                 \
  hipLaunchKernelGGL((k_decode_split<D>), dim3(ns, Hkv, B), dim3(kThreads), 0, s, l,                  \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_h,                            \
                     (const unsigned short*)k_cache.ptr, k_cache.stride_b, k_cache.stride_t,          \
                     k_cache.stride_h, (const unsigned short*)v_cache.ptr, v_cache.stride_b,          \
                     v_cache.stride_t, v_cache.stride_h, Hq, Hkv, kv_len, sel, sel_groups, c2, w, ns)
#define GSA_COMBINE(D, TO)                                                                           \
  hipLaunchKernelGGL((k_decode_combine<D, TO>), dim3(Hq, B), dim3(D), 0, s, w, Hq, Hkv, ns,           \
                     (TO*)o.ptr, o.stride_b, o.stride_h, lse)
  if (d == 128) {
    GSA_SPLIT(128);
    if ((st = launch_status("gsa_attn_decode (split)")) != GSA_OK) return st;
    if (o.dtype == GSA_F32) GSA_COMBINE(128, float);
    else GSA_COMBINE(128, unsigned short);
  } else {
    GSA_SPLIT(64);
    if ((st = launch_status("gsa_attn_decode (split)")) != GSA_OK) return st;
    if (o.dtype == GSA_F32) GSA_COMBINE(64, float);
    else GSA_COMBINE(64, unsigned short);
  }
#undef GSA_SPLIT
#undef GSA_COMBINE
  return launch_status("gsa_attn_decode (combine)");
}
