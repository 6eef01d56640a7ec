// Fixed-layout decode over a compacted KV cache: real removal of the raw
// tokens that have left the local window.
//
// With the fixed layout (no unfolding) a query only ever sees the sinks, every
// gist and its local window (UniGist summary, Approach), so a cache for it
// need not keep raw tokens older than the window: UniGist's summary reports
// actually removing the compressed tokens at inference, and the Study page
// (§2 Preliminaries) puts the saving at 75% of the KV memory for ratio 4.  The
// compact cache of one (batch, KV head) is
//   [ S sink slots | gist_capacity gist slots | W ring slots ]
// where the t-th gist of the sequence lives in gist slot t and a raw token at
// position p in ring slot p mod W (W = max(window, 1)); a raw token is
// overwritten W positions later, by which time no query can see it.
//
// gsa_compact_append writes new tokens' K/V into their slots;
// gsa_compact_decode attends one query per sequence (position `pos`) to the
// sinks, the gists at or before it and the raws of its window -- the same set
// as the fixed layout over the full cache -- with the split-K streaming of the
// fused decode step.
#include "decode_stream.h"

namespace gsa {
namespace {
using namespace dec;

struct CompactArgs {
  Lay l;
  int gcap;                             // gist slots
  const unsigned short* q;
  int64_t qsb, qsh;
  const unsigned short* kc;
  int64_t ksb, kst, ksh;
  const unsigned short* vc;
  int64_t vsb, vst, vsh;
  int Hq, Hkv, pos;
  float c2;
  int* counters;                        // [B*Hkv]
  float* part;                          // [B*Hkv][ns][G][D + kPartExtra]
  int ns, rp;
  void* o;
  int64_t osb, osh;
  float* lse;
};

// Slot of sequence position p (single level).
__device__ inline int compact_slot(const Lay& l, int gcap, int p) {
  if (p < l.S) return p;
  const int y = p - l.S;
  const int f = fdiv(l.dP, y), r = y - f * l.P;
  if (r >= l.c) return l.S + f * l.g + (r - l.c);    // gist number f*g + (r - c)
  return l.S + gcap + p % l.W1;                      // raw: ring slot
}

template <int D, typename TO>
__global__ __launch_bounds__(kThreads) void k_compact_decode(CompactArgs a) {
  using C = DCfg<D>;
  const Lay& l = a.l;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const int i = a.pos;
  const int lo = imax(0, i - l.W1 + 1);
  const size_t gidx = (size_t)b * a.Hkv + h;
  // visible rows: [sinks | gists at or before i | raws of the window]
  const int nsink = imin(l.S, i + 1);
  const int ngist = count_below(l, K_GIST, i + 1);
  const int r_lo = count_below(l, K_RAW, lo), r_hi = count_below(l, K_RAW, i + 1);
  const int total = nsink + ngist + (r_hi - r_lo);

  __shared__ __attribute__((aligned(1024))) StepLds<D> lds;
  __shared__ int rowpos[2][kRows], rowflag[3][kRows];
  __shared__ float wstat[192];
  __shared__ int am_last;

  bf16x8 qreg[C::KS];
  {
    const unsigned short* qrow = a.q + b * a.qsb + (int64_t)(h * G + imin(col, G - 1)) * a.qsh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * grp + 32 * ks);
      if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  auto info = [&](int v, int& slot, int& fl) {
    fl = kAttend;
    if (v < nsink) {
      slot = v;
    } else if (v < nsink + ngist) {
      slot = l.S + (v - nsink);
    } else {
      const int p = pos_of(l, K_RAW, r_lo + (v - nsink - ngist));
      slot = l.S + a.gcap + p % l.W1;
    }
  };
  const unsigned short* kb = a.kc + b * a.ksb + h * a.ksh;
  const unsigned short* vb = a.vc + b * a.vsb + h * a.vsh;
  const int v_begin = imin(split * a.rp, total);
  const int v_end = imin(v_begin + a.rp, total);
  f32x4 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f, l_ex = 0.f;
  stream_rows<D>(v_begin, v_end, info, kb, a.kst, vb, a.vst, qreg, a.c2, lds.stage0, lds.stage1, rowpos, rowflag,
                 nullptr, oacc, m_run, l_run, l_ex);
  constexpr int PS = D + kPartExtra;
  float* gpart = a.part + gidx * a.ns * G * PS;
  store_partial<D>(oacc, m_run, l_run, l_ex, G, wstat, reinterpret_cast<float*>(lds.stage0),
                   gpart + (size_t)split * G * PS);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&a.counters[gidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    am_last = prev == a.ns - 1;
  }
  __syncthreads();
  if (!am_last) return;
  merge_partials<D, TO>(gpart, a.ns, G, reinterpret_cast<TO*>(a.o), a.osb, a.osh, a.lse, a.Hq, b, h);
  if (tid == 0) __hip_atomic_store(&a.counters[gidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per (new token, KV head, batch): copies the token's K and V
// rows into its slot.  Raw tokens that would already be out of the window of
// the last appended position are skipped, so no two tokens of one call share
// a ring slot.
__global__ __launch_bounds__(64) void k_compact_append(Lay l, int gcap, const unsigned short* __restrict__ kn,
                                                       int64_t knb, int64_t knt, int64_t knh,
                                                       const unsigned short* __restrict__ vn, int64_t vnb,
                                                       int64_t vnt, int64_t vnh, int pos0, int n, int d,
                                                       unsigned short* __restrict__ kc, int64_t ksb, int64_t kst,
                                                       int64_t ksh, unsigned short* __restrict__ vc, int64_t vsb,
                                                       int64_t vst, int64_t vsh) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int p = pos0 + t;
  const int slot = compact_slot(l, gcap, p);
  const bool ring = slot >= l.S + gcap;
  if (ring && p <= pos0 + n - 1 - l.W1) return;   // out of every later window
  const u32x4* ks = reinterpret_cast<const u32x4*>(kn + b * knb + t * knt + h * knh);
  const u32x4* vs = reinterpret_cast<const u32x4*>(vn + b * vnb + t * vnt + h * vnh);
  u32x4* kd = reinterpret_cast<u32x4*>(kc + b * ksb + (int64_t)slot * kst + h * ksh);
  u32x4* vd = reinterpret_cast<u32x4*>(vc + b * vsb + (int64_t)slot * vst + h * vsh);
  for (int e = threadIdx.x; e < d / 8; e += 64) {
    kd[e] = ks[e];
    vd[e] = vs[e];
  }
}

gsa_status compact_layout(const gsa_layout* layout, int len, Lay* l) {
  gsa_status st = make_lay(layout, len, 64, l);
  if (st != GSA_OK) return st;
  if (l->k != 0 || l->G2 != 0)
    return fail(GSA_EUNSUPPORTED, "the compact cache is for the fixed layout (top_k = 0, one level): unfolding "
                                  "needs raw tokens that the compact cache has removed");
  return GSA_OK;
}

struct CompactPlan {
  int ns, rp;
  size_t off_part, bytes;
};

void plan_compact(const Lay& l, int B, int Hq, int Hkv, int d, int pos, CompactPlan* p) {
  const int i = pos;
  const int lo = imax(0, i - l.W1 + 1);
  const int rows = imin(l.S, i + 1) + count_below(l, K_GIST, i + 1) + count_below(l, K_RAW, i + 1) -
                   count_below(l, K_RAW, lo);
  const int groups = imax(1, B * Hkv);
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  int ns = iclamp((2 * cus + groups - 1) / groups, 1, kMaxSplit);
  ns = imin(ns, imax(1, (rows + kRows - 1) / kRows));
  p->rp = imax(kRows, ((rows + ns - 1) / ns + kRows - 1) / kRows * kRows);
  p->ns = imax(1, (rows + p->rp - 1) / p->rp);
  p->off_part = ((size_t)groups * sizeof(int) + 255) / 256 * 256;
  p->bytes = p->off_part + (size_t)groups * p->ns * (Hq / Hkv) * (d + kPartExtra) * sizeof(float);
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" int32_t gsa_compact_slots(const gsa_layout* layout, int32_t gist_capacity) {
  Lay l;
  if (compact_layout(layout, 0, &l) != GSA_OK || gist_capacity < 0) return -1;
  return l.S + gist_capacity + l.W1;
}

extern "C" int32_t gsa_compact_gists(const gsa_layout* layout, int32_t seq_len) {
  Lay l;
  if (compact_layout(layout, seq_len, &l) != GSA_OK) return -1;
  return count_below(l, K_GIST, seq_len);
}

extern "C" gsa_status gsa_compact_append(const gsa_layout* layout, gsa_tensor k_new, gsa_tensor v_new, int32_t B,
                                         int32_t Hkv, int32_t d, int32_t pos0, int32_t n, gsa_tensor k_cache,
                                         gsa_tensor v_cache, int32_t gist_capacity, void* stream) {
  Lay l;
  gsa_status st = compact_layout(layout, pos0 + n, &l);
  if (st != GSA_OK) return st;
  if ((st = check_tensor("k_new", k_new, d)) != GSA_OK) return st;
  if ((st = check_tensor("v_new", v_new, d)) != GSA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, d)) != GSA_OK) return st;
  if (k_new.dtype != GSA_BF16 || v_new.dtype != GSA_BF16 || k_cache.dtype != GSA_BF16 || v_cache.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "the compact cache holds bf16");
  if (B < 1 || Hkv < 1) return fail(GSA_EINVAL, "bad sizes B=%d Hkv=%d", B, Hkv);
  if (d < 8 || d % 8 || d > 512) return fail(GSA_EUNSUPPORTED, "head dim %d", d);
  if (pos0 < 0 || n < 0) return fail(GSA_EINVAL, "positions [%d, %d)", pos0, pos0 + n);
  if (gist_capacity < 0) return fail(GSA_EINVAL, "gist_capacity %d < 0", gist_capacity);
  if (count_below(l, K_GIST, pos0 + n) > gist_capacity)
    return fail(GSA_EINVAL, "positions up to %d hold %d gists, more than the %d gist slots", pos0 + n - 1,
                count_below(l, K_GIST, pos0 + n), gist_capacity);
  if (n == 0) return GSA_OK;
  hipLaunchKernelGGL(k_compact_append, dim3(n, Hkv, B), dim3(64), 0, (hipStream_t)stream, l, gist_capacity,
                     (const unsigned short*)k_new.ptr, k_new.stride_b, k_new.stride_t, k_new.stride_h,
                     (const unsigned short*)v_new.ptr, v_new.stride_b, v_new.stride_t, v_new.stride_h, pos0, n, d,
                     (unsigned short*)k_cache.ptr, k_cache.stride_b, k_cache.stride_t, k_cache.stride_h,
                     (unsigned short*)v_cache.ptr, v_cache.stride_b, v_cache.stride_t, v_cache.stride_h);
  return launch_status("gsa_compact_append");
}

extern "C" size_t gsa_compact_decode_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                                     int32_t d, int32_t pos) {
  Lay l;
  if (compact_layout(layout, pos + 1, &l) != GSA_OK || pos < 0 || B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv) return 0;
  CompactPlan p;
  plan_compact(l, B, Hq, Hkv, d, pos, &p);
  return p.bytes;
}

extern "C" gsa_status gsa_compact_decode(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                                         gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t pos, int32_t gist_capacity, float scale,
                                         void* ws, size_t ws_bytes, void* stream) {
  Lay l;
  gsa_status st = compact_layout(layout, pos + 1, &l);
  if (st != GSA_OK) return st;
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("o", o, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k_cache.dtype != GSA_BF16 || v_cache.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "compact decode takes bf16 q and caches");
  if (o.dtype != GSA_F32 && o.dtype != GSA_BF16) return fail(GSA_EINVAL, "o dtype");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (Hq / Hkv > 16) return fail(GSA_EUNSUPPORTED, "more than 16 query heads per KV head");
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (pos < 0) return fail(GSA_EINVAL, "pos %d < 0", pos);
  if (count_below(l, K_GIST, pos + 1) > gist_capacity)
    return fail(GSA_EINVAL, "position %d needs %d gist slots (capacity %d)", pos, count_below(l, K_GIST, pos + 1),
                gist_capacity);
  CompactPlan p;
  plan_compact(l, B, Hq, Hkv, d, pos, &p);
  if (!ws || ws_bytes < p.bytes) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", p.bytes, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GSA_EINVAL, "workspace must be 256-byte aligned");
  CompactArgs a;
  a.l = l;
  a.gcap = gist_capacity;
  a.q = (const unsigned short*)q.ptr;
  a.qsb = q.stride_b;
  a.qsh = q.stride_h;
  a.kc = (const unsigned short*)k_cache.ptr;
  a.ksb = k_cache.stride_b;
  a.kst = k_cache.stride_t;
  a.ksh = k_cache.stride_h;
  a.vc = (const unsigned short*)v_cache.ptr;
  a.vsb = v_cache.stride_b;
  a.vst = v_cache.stride_t;
  a.vsh = v_cache.stride_h;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.pos = pos;
  a.c2 = scale * kLog2e;
  a.counters = (int*)ws;
  a.part = (float*)((char*)ws + p.off_part);
  a.ns = p.ns;
  a.rp = p.rp;
  a.o = o.ptr;
  a.osb = o.stride_b;
  a.osh = o.stride_h;
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(p.ns, Hkv, B);
  if (d == 128) {
    if (o.dtype == GSA_F32) hipLaunchKernelGGL((k_compact_decode<128, float>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_compact_decode<128, unsigned short>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (o.dtype == GSA_F32) hipLaunchKernelGGL((k_compact_decode<64, float>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_compact_decode<64, unsigned short>), grid, dim3(kThreads), 0, s, a);
  }
  return launch_status("gsa_compact_decode");
}
