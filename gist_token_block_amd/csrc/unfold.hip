// Selective unfolding at prefill scale: the raw tokens of each query's chosen
// chunks (Simplified Sparse Attention via Gist Tokens, abstract: unfold the
// top-k chunks by reintroducing their raw tokens; Forget, Then Recall ... Gist
// Sparse Attention, abstract: restore the raw chunks of the selected gists).
//
// A query's visible keys split into two disjoint parts:
//   * the fixed part -- sinks, every gist at or before it, its window -- which
//     is the same block-sparse pattern for every query and runs on the MFMA
//     prefill over the fixed layout's tile table;
//   * the unfolded raws -- the raw tokens of its k chosen chunks that lie
//     before the window (those inside it are already in the fixed part) --
//     which differ from query to query.
// k_unfold attends each query to its unfolded raws (one wave per query and KV
// group: the G query heads share the selection) and leaves a softmax partial
// (unnormalised O, running max, sums) per query head; the prefill kernel then
// starts each row from that partial instead of from zero, so the result is the
// softmax over the union with no second pass and no double rounding.
#include "gsa_internal.h"
#include "select_net.h"

namespace gsa {

// Floats per (query, head) partial: O (d floats), max (log2 units), sum of
// the probabilities, sum again (the log-sum-exp's, identical here: fp32 P).
constexpr int kUnfoldExtra = 3;

namespace {

constexpr int kWaves = 4;
constexpr int kMaxKeys = 64;       // unfolded raws handled per pass of a wave
constexpr int kMaxG = 16;

// One wave per (batch, KV head, query row), grid-stride; MG bounds the query
// heads per KV head (the per-head registers are sized by it).  Lane j of a pass
// owns unfolded key j: it computes that key's logits for the group's heads; the
// probabilities go through LDS, and each lane then accumulates two output
// dimensions over the pass's keys.
template <int D, int MG>
__global__ __launch_bounds__(64 * kWaves) void k_unfold(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh, int B, int Hq, int Hkv,
    int q_begin, int q_len, const int* __restrict__ sel, float c2, float* __restrict__ part) {
  constexpr int PS = D + kUnfoldExtra;
  constexpr int DPL = D / 64;      // output dimensions per lane
  __shared__ float qs[kWaves][MG][D];
  __shared__ float ps[kWaves][MG][kMaxKeys];
  __shared__ int kpos[kWaves][kMaxKeys];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = Hq / Hkv;
  const long long total = (long long)B * Hkv * q_len;
  for (long long item = (long long)blockIdx.x * kWaves + wave; item < total; item += (long long)gridDim.x * kWaves) {
    const int r = (int)(item % q_len);
    const int h = (int)((item / q_len) % Hkv);
    const int b = (int)(item / ((long long)q_len * Hkv));
    const int i = q_begin + r;
    const int lo = imax(0, i - l.W1 + 1);
    const int nch = count_below(l, K_GIST, i) / l.g;   // complete chunks
    // this query's unfolded raws: chunk e's raws before the window, laid out
    // by an exclusive scan over the selection
    int len = 0, st = 0;
    if (lane < l.k) {
      const int m = sel[(((size_t)b * Hkv + h) * q_len + r) * l.k + lane];
      if (m >= 0 && m < nch) {
        st = pos_of(l, K_RAW, m * l.c);
        len = iclamp(lo - st, 0, l.c);
      }
    }
    int incl = len;
#pragma unroll
    for (int j = 1; j < 64; j <<= 1) {
      const int t = __shfl_up(incl, j);
      if (lane >= j) incl += t;
    }
    const int nk = __shfl(incl, 63);
    const int excl = incl - len;
    // query rows of the group, as fp32, into LDS
    for (int x = lane; x < G * D; x += 64) {
      const int hd = x / D, dd = x - hd * D;
      qs[wave][hd][dd] = bf16_to_f32(q[b * qsb + (int64_t)r * qst + (int64_t)(h * G + hd) * qsh + dd]);
    }
    float m_run[MG], l_run[MG], acc[MG][DPL];
#pragma unroll
    for (int hd = 0; hd < MG; ++hd) {
      m_run[hd] = kNegBig;
      l_run[hd] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hd][e] = 0.f;
    }
    for (int k0 = 0; k0 < nk; k0 += kMaxKeys) {
      // position of key k0 + lane: the run (chunk) holding it.  When every
      // chosen chunk unfolds whole (k c keys), key x is raw x % c of chunk x / c.
      int p = -1;
      const int kk = k0 + lane;
      if (nk == l.k * l.c) {
        const int e = kk / l.c;
        const int st_e = __shfl(st, imin(e, 63));
        if (kk < nk) p = st_e + (kk - e * l.c);
      } else {
        for (int e = 0; e < l.k && e < 64; ++e) {
          const int s_e = __shfl(excl, e), l_e = __shfl(len, e), st_e = __shfl(st, e);
          if (kk >= s_e && kk < s_e + l_e) p = st_e + (kk - s_e);
        }
      }
      kpos[wave][lane] = p;
      __builtin_amdgcn_wave_barrier();
      // logits of key lane for every head of the group: the whole K row is
      // loaded first (all its pieces in flight), then dotted with the group's
      // query rows read from LDS as broadcasts
      float lg[MG];
#pragma unroll
      for (int hd = 0; hd < MG; ++hd) lg[hd] = 0.f;
      {
        u32x4 kr[D / 8];
        const unsigned short* krow = k + b * ksb + (int64_t)imax(p, 0) * kst + h * ksh;
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8)
          kr[c8] = p >= 0 ? *reinterpret_cast<const u32x4*>(krow + 8 * c8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int hd = 0; hd < MG; ++hd) {
          if (hd < G) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) {
              const f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[wave][hd][8 * c8]);
              const f32x4 qb = *reinterpret_cast<const f32x4*>(&qs[wave][hd][8 * c8 + 4]);
              const u32x4 w = kr[c8];
              a0 = fmaf(qa[0], lo_bf16(w[0]), a0);
              a1 = fmaf(qa[1], hi_bf16(w[0]), a1);
              a0 = fmaf(qa[2], lo_bf16(w[1]), a0);
              a1 = fmaf(qa[3], hi_bf16(w[1]), a1);
              a0 = fmaf(qb[0], lo_bf16(w[2]), a0);
              a1 = fmaf(qb[1], hi_bf16(w[2]), a1);
              a0 = fmaf(qb[2], lo_bf16(w[3]), a0);
              a1 = fmaf(qb[3], hi_bf16(w[3]), a1);
            }
            lg[hd] = a0 + a1;
          }
        }
      }
      // online softmax per head over this pass's keys (base 2)
#pragma unroll
      for (int hd = 0; hd < MG; ++hd) {
        if (hd < G) {
          const float s = p >= 0 ? lg[hd] * c2 : -__builtin_inff();
          float mx = s;
#pragma unroll
          for (int j = 32; j > 0; j >>= 1) mx = fmaxf(mx, xor_lane(mx, j));
          const float m_new = fmaxf(m_run[hd], mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run[hd] - m_new);
          const float pr = p >= 0 ? __builtin_amdgcn_exp2f(s - m_new) : 0.f;
          float sum = pr;
#pragma unroll
          for (int j = 32; j > 0; j >>= 1) sum += xor_lane(sum, j);
          l_run[hd] = l_run[hd] * alpha + sum;
          m_run[hd] = m_new;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[hd][e] *= alpha;
          ps[wave][hd][lane] = pr;
        }
      }
      __builtin_amdgcn_wave_barrier();
      // PV: lane owns output dimensions lane * DPL .. + DPL - 1; every V load
      // of the pass is issued before the products
      const int nkp = imin(kMaxKeys, nk - k0);
      unsigned vw[kMaxKeys];
#pragma unroll
      for (int j = 0; j < kMaxKeys; ++j) {
        vw[j] = 0u;
        if (j < nkp) {
          const int pj = kpos[wave][j];
          const unsigned short* vrow = v + b * vsb + (int64_t)pj * vst + h * vsh + lane * DPL;
          if constexpr (DPL == 2) vw[j] = *reinterpret_cast<const unsigned*>(vrow);
          else vw[j] = (unsigned)vrow[0] << 16;
        }
      }
#pragma unroll
      for (int j4 = 0; j4 < kMaxKeys; j4 += 4) {
        if (j4 < nkp) {
#pragma unroll
          for (int hd = 0; hd < MG; ++hd) {
            if (hd < G) {
              const f32x4 pr = *reinterpret_cast<const f32x4*>(&ps[wave][hd][j4]);
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                if constexpr (DPL == 2) {
                  acc[hd][0] = fmaf(pr[jj], lo_bf16(vw[j4 + jj]), acc[hd][0]);
                  acc[hd][1] = fmaf(pr[jj], hi_bf16(vw[j4 + jj]), acc[hd][1]);
                } else {
                  acc[hd][0] = fmaf(pr[jj], hi_bf16(vw[j4 + jj]), acc[hd][0]);
                }
              }
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // the partial of each head: unnormalised O, max (log2 units), sums
#pragma unroll
    for (int hd = 0; hd < MG; ++hd) {
      if (hd < G) {
        float* dst = part + (((size_t)b * q_len + r) * Hq + h * G + hd) * PS;
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[lane * DPL + e] = acc[hd][e];
        if (lane == 0) {
          dst[D] = m_run[hd];
          dst[D + 1] = l_run[hd];
          dst[D + 2] = l_run[hd];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

gsa_status launch_unfold(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k, const gsa_tensor& v, int B,
                         int Hq, int Hkv, int q_begin, int q_len, const int* sel, float scale, float* part,
                         hipStream_t st) {
  if (Hq / Hkv > kMaxG) return fail(GSA_EUNSUPPORTED, "more than %d query heads per KV head", kMaxG);
  if (l.k > 64) return fail(GSA_EUNSUPPORTED, "top_k %d > 64", l.k);
  const long long items = (long long)B * Hkv * q_len;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const long long want = (items + kWaves - 1) / kWaves;
  const int grid = (int)(want < 8LL * cus ? want : 8LL * cus);
  const float c2 = scale * kLog2e;
#define GSA_UNFOLD2(D, MG)                                                                              \
  hipLaunchKernelGGL((k_unfold<D, MG>), dim3(grid), dim3(64 * kWaves), 0, st, l, (const unsigned short*)q.ptr, \
                     q.stride_b, q.stride_t, q.stride_h, (const unsigned short*)k.ptr, k.stride_b,         \
                     k.stride_t, k.stride_h, (const unsigned short*)v.ptr, v.stride_b, v.stride_t,         \
                     v.stride_h, B, Hq, Hkv, q_begin, q_len, sel, c2, part)
#define GSA_UNFOLD(D)                              \
  do {                                             \
    if (Hq / Hkv <= 4) GSA_UNFOLD2(D, 4);          \
    else if (Hq / Hkv <= 8) GSA_UNFOLD2(D, 8);     \
    else GSA_UNFOLD2(D, 16);                       \
  } while (0)
  if (d == 128) GSA_UNFOLD(128);
  else if (d == 64) GSA_UNFOLD(64);
  else return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
#undef GSA_UNFOLD
#undef GSA_UNFOLD2
  return launch_status("gsa_attn_prefill_unfolded (unfold)");
}

}  // namespace gsa
