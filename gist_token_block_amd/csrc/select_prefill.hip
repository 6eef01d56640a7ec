// Per-row top-k selection at prefill scale (gsa_select_prefill): every query
// row scores every chunk whose gist precedes it against the gist key only,
// and keeps the k best (Simplified Sparse Attention via Gist Tokens, abstract;
// the score of a chunk for one KV head is the mean over that KV group's query
// heads of q.k * scale; ties go to the lower chunk index).  The ranking is the
// ranking of the plain sum over the group's heads of q.k: mean and scale are
// positive factors.
//
// One workgroup per (batch, KV head, 128 query rows); wave w owns rows
// [32w, 32w + 32) as the N dimension of v_mfma_f32_32x32x16_bf16, and the
// gist stream goes through LDS in 64-key tiles (double buffered, straight
// from HBM/L2 with global_load_lds), exactly as the prefill streams K.
//   * Scores: S^T = K_gist qsum^T, where qsum (the sum of the group's query
//     heads, formed exactly in fp32) is split into two bf16 parts hi + lo and
//     both go through the MFMA: bf16 x bf16 products are exact and the sum is
//     fp32, so a score carries fp32 rounding of the products' sum plus the
//     split's residual (2^-17 of |qsum| per element) -- the accuracy of a plain
//     fp32 dot product for ranking purposes.
//   * Each lane owns half the candidates of one row and keeps its best KA >= k
//     as sorted 64-bit keys.  Per tile it marks the candidates that reach the
//     larger of its own and its partner lane's current worst (a candidate below
//     a full list of the same row cannot be in the row's best KA), then inserts
//     each marked one, re-checked exactly, once per trip.
//   * The two lanes of a row merge their lists; the k best are written in
//     ascending chunk order.
#include <limits.h>

#include "gsa_internal.h"
#include "select_net.h"

namespace gsa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* glb_void_ptr;

template <int D> struct SCfg {
  static constexpr int PPR = D / 8;
  static constexpr int RPI = 64 / PPR;
  static constexpr int NIW = kBN / RPI / 4;
  static constexpr int KS = D / 16;
};
template <int D> __device__ inline int sswz(int r) { return r & (D / 8 - 1); }

// A score as an unsigned word with the order of the floats (negative scores
// flipped whole, positive ones get the sign bit): -inf maps to 0x007fffff, so
// 0 stands for an empty slot below every real score.  Scores are never NaN
// here (a NaN score ranks as -inf).  With ~id below it, a 64-bit key orders
// like (score desc, id asc).
__device__ inline unsigned mono(float s) {
  const unsigned u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float unmono(unsigned m) { return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m); }
__device__ inline unsigned long long make_key(unsigned m, int id) {
  return m ? ((unsigned long long)m << 32) | (unsigned)~id : 0ull;
}
__device__ inline int key_id(unsigned long long k) { return (int)~(unsigned)k; }
// median of three words (the middle one of a <= c and any b)
__device__ inline unsigned umed3(unsigned a, unsigned b, unsigned c) {
  unsigned r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline unsigned partner_word(unsigned v, int h2) {
  const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return h2 ? sw[0] : sw[1];
}

template <int D, int KA>
__global__ __launch_bounds__(kThreads, 2) void k_select_prefill(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh, int Hq, int Hkv, int q_begin,
    int q_len, int nqt, int total, int* __restrict__ sel) {
  using C = SCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned short K0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short K1[kBN * D];
  __shared__ float sc[4][32][64];           // a wave's tile scores: [slot][lane]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  // XCD-aware order: each XCD (blockIdx % 8) runs a contiguous range of
  // (batch, KV head, query tile descending), so the workgroups sharing one KV
  // head's gist stream share an L2 and the heaviest tiles start first.
  const int x = blockIdx.x;
  const int per = total >> 3, rem = total & 7, xcd = x & 7;
  const int logical = xcd * per + imin(xcd, rem) + (x >> 3);
  const int qt = nqt - 1 - logical % nqt;
  const int h = (logical / nqt) % Hkv, b = logical / nqt / Hkv;
  const int G = Hq / Hkv;
  const int r = qt * kBM + wave * 32 + n;
  const bool rvalid = r < q_len;
  const int rr = imin(r, q_len - 1);
  const int i = q_begin + rr;
  const int ncand = count_below(l, K_GIST, i);                 // one gist per chunk
  const int r_last = imin(qt * kBM + kBM - 1, q_len - 1);
  const int ncand_max = count_below(l, K_GIST, q_begin + r_last);
  const int ngist_all = imax(1, count_below(l, K_GIST, l.L));
  const int ntile = (ncand_max + kBN - 1) / kBN;

  // qsum^T operands as bf16 hi + lo: lane (n, h2) holds d = 8 h2 + 16 ks + 0..7
  bf16x8 qhi[C::KS], qlo[C::KS];
  {
    const unsigned short* q0 = q + b * qsb + (int64_t)rr * qst + (int64_t)(h * G) * qsh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int g = 0; g < G; ++g) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(q0 + (int64_t)g * qsh + 8 * h2 + 16 * ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[2 * e] += lo_bf16(w[e]);
          a[2 * e + 1] += hi_bf16(w[e]);
        }
      }
      u32x4 ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = pack_bf16x2(a[2 * e], a[2 * e + 1]);
        pl[e] = pack_bf16x2(a[2 * e] - lo_bf16(ph[e]), a[2 * e + 1] - hi_bf16(ph[e]));
      }
      qhi[ks] = __builtin_bit_cast(bf16x8, ph);
      qlo[ks] = __builtin_bit_cast(bf16x8, pl);
    }
  }

  const unsigned short* kb = k + b * ksb + h * ksh;
  const int srow = lane / C::PPR, sslot = lane % C::PPR;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto fetch = [&](int t, unsigned short* Kd) {
#pragma unroll
    for (int it = 0; it < C::NIW; ++it) {
      const int wi = wv * C::NIW + it;
      const int row = wi * C::RPI + srow;
      const int u = imin(t * kBN + row, ngist_all - 1);
      const int p = pos_of(l, K_GIST, u);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(kb + (int64_t)p * kst + 8 * (sslot ^ sswz<D>(row))),
                                       (lds_void_ptr)(Kd + wi * 512), 16, 0, 0);
    }
  };
  int qk_off[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qk_off[ks] = n * D + 8 * ((h2 + 2 * ks) ^ sswz<D>(n));
    asm volatile("" : "+v"(qk_off[ks]));
  }

  // The lane's survivors, ascending (slot 0 is the worst): km the order-
  // preserving words of their scores (0: empty), ki their ids.  Candidates
  // reach a lane in ascending id order, so a newcomer ranks below every
  // survivor of equal score and beats a slot exactly when its word is larger.
  unsigned km[KA];
  int ki[KA];
#pragma unroll
  for (int j = 0; j < KA; ++j) {
    km[j] = 0u;
    ki[j] = 0;
  }

  if (ntile > 0) fetch(0, K0);
  auto tile = [&](int t, const unsigned short* Kb, unsigned short* Kn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntile) fetch(t + 1, Kn);
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Kb + qk_off[ks]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(Kb + qk_off[ks] + 32 * D);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qhi[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qhi[ks], s1, 0, 0, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qlo[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qlo[ks], s1, 0, 0, 0);
    }
    // value slot x = 16 half + j is candidate 64 t + 32 half + 8 (j / 4) + 4 h2 + j % 4.
    // Threshold: the larger of the two lanes' worst survivors, counting a
    // list only when full.  The mask marks a superset of the candidates that
    // can still enter (score >= threshold; every candidate while neither list
    // bounds it, NaN included, which ranks as -inf); each marked one is
    // re-checked exactly before it is inserted.
    const unsigned pw = partner_word(km[0], h2);
    const float own = km[0] ? unmono(km[0]) : -__builtin_inff();
    const float oth = pw ? unmono(pw) : -__builtin_inff();
    const float thr = fmaxf(own, oth);
    unsigned mask = 0;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      const float v = x < 16 ? s0[x & 15] : s1[x & 15];
      sc[wave][x][lane] = v;
      mask |= (unsigned)(v >= thr) << x;
    }
    if (thr == -__builtin_inff()) mask = 0xffffffffu;
    if (!rvalid) mask = 0u;
    const int idb = t * kBN + 4 * h2;
    // one sorted insertion per marked candidate and trip, straight-line in
    // every lane (a lane with nothing left inserts the empty key: no change).
    // The empty asm statements keep the read and the key opaque, so the
    // compiler neither predicates the read nor turns the uniform loop into a
    // per-lane one (which copies every key at each trip).
    int most = __popc(mask);   // trips: the largest count of marks in the wave
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) most = imax(most, xor_lane(most, o));
    const int trips = __builtin_amdgcn_readfirstlane(most);
    for (int trip = 0; trip < trips; ++trip) {
      const bool has = mask != 0u;
      const int xs = has ? __builtin_ctz(mask) : 0;
      mask &= mask - 1u;
      float sv = sc[wave][xs][lane];
      asm volatile("" : "+v"(sv));
      const int j = xs & 15;
      const int id = idb + 32 * (xs >> 4) + 8 * (j >> 2) + (j & 3);
      unsigned m = mono(nan_to_neg_inf(sv));
      asm volatile("" : "+v"(m));
      unsigned cm = (has && id < ncand) ? m : 0u;
      asm volatile("" : "+v"(cm));
      bool gt_next = cm > km[0];
#pragma unroll
      for (int e = 0; e < KA - 1; ++e) {
        const bool gt_e = gt_next;
        gt_next = cm > km[e + 1];
        ki[e] = gt_next ? ki[e + 1] : (gt_e ? id : ki[e]);
        km[e] = umed3(km[e], cm, km[e + 1]);
      }
      ki[KA - 1] = gt_next ? id : ki[KA - 1];
      km[KA - 1] = gt_next ? cm : km[KA - 1];
    }
  };
  for (int t = 0; t < ntile; t += 2) {
    tile(t, K0, K1);
    if (t + 1 < ntile) tile(t + 1, K1, K0);
  }

  // ---- the row's best KA of both lists: with both ascending, the larger of
  // own[j] and partner[KA - 1 - j] over j are the KA best of the union
  unsigned long long best[KA];
#pragma unroll
  for (int j = 0; j < KA; ++j) {
    const unsigned long long mine = make_key(km[j], ki[j]);
    const unsigned long long o = make_key(partner_word(km[KA - 1 - j], h2), partner_word(ki[KA - 1 - j], h2));
    best[j] = mine > o ? mine : o;
  }
  if (!rvalid || h2 != 0) return;
  // rank among them (0 = best); the k best that exist are chosen and written
  // at their place in ascending chunk order, -1 after them
  int* out = sel + (((size_t)b * Hkv + h) * q_len + r) * l.k;
  int nchosen = 0;
  bool chosen[KA];
#pragma unroll
  for (int j = 0; j < KA; ++j) {
    int rank = 0;
#pragma unroll
    for (int u = 0; u < KA; ++u) rank += best[u] > best[j] ? 1 : 0;
    chosen[j] = best[j] != 0ull && rank < l.k;
    nchosen += chosen[j] ? 1 : 0;
  }
#pragma unroll
  for (int j = 0; j < KA; ++j) {
    if (!chosen[j]) continue;
    const int id = key_id(best[j]);
    int pos = 0;
#pragma unroll
    for (int u = 0; u < KA; ++u) pos += (chosen[u] && key_id(best[u]) < id) ? 1 : 0;
    out[pos] = id;
  }
  for (int t = nchosen; t < l.k; ++t) out[t] = -1;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status gsa_select_prefill(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, int32_t B,
                                         int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len, int32_t q_begin,
                                         int32_t q_len, float scale, int32_t* sel, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, kBN, &l);
  if (st != GSA_OK) return st;
  if (l.G2 != 0) return fail(GSA_EUNSUPPORTED, "gsa_select_prefill takes one level (gsa_score_select does two)");
  if (l.g != 1) return fail(GSA_EUNSUPPORTED, "gsa_select_prefill takes one gist per chunk (gsa_score_select any)");
  if (l.k < 1 || l.k > 32) return fail(GSA_EUNSUPPORTED, "top_k %d outside [1, 32]", l.k);
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k", k, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k.dtype != GSA_BF16) return fail(GSA_EUNSUPPORTED, "gsa_select_prefill takes bf16");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (d != 128 && d != 64) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  const int nqt = (q_len + kBM - 1) / kBM;
  const long long total = (long long)B * Hkv * nqt;
  if (total > 0x7fffffff) return fail(GSA_EUNSUPPORTED, "grid too large");
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)total);
#define GSA_SEL(D, KA)                                                                                      \
  hipLaunchKernelGGL((k_select_prefill<D, KA>), grid, dim3(kThreads), 0, s, l, (const unsigned short*)q.ptr, \
                     q.stride_b, q.stride_t, q.stride_h, (const unsigned short*)k.ptr, k.stride_b, k.stride_t,  \
                     k.stride_h, Hq, Hkv, q_begin, q_len, nqt, (int)total, sel)
  if (d == 128) {
    if (l.k <= 8) GSA_SEL(128, 8);
    else if (l.k <= 16) GSA_SEL(128, 16);
    else GSA_SEL(128, 32);
  } else {
    if (l.k <= 8) GSA_SEL(64, 8);
    else if (l.k <= 16) GSA_SEL(64, 16);
    else GSA_SEL(64, 32);
  }
#undef GSA_SEL
  return launch_status("gsa_select_prefill");
}
