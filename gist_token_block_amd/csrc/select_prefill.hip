// Per-row top-k selection at prefill scale (gsa_select_prefill): every query
// row scores every chunk whose gist precedes it against the gist key only,
// and keeps the k best (Simplified Sparse Attention via Gist Tokens, abstract;
// the score of a chunk for one KV head is the mean over that KV group's query
// heads of q.k * scale; ties go to the lower chunk index).
//
// One workgroup per (batch, KV head, 128 query rows); wave w owns rows
// [32w, 32w + 32) as the N dimension of v_mfma_f32_32x32x16_bf16, and the
// gist stream goes through LDS in 64-key tiles (double buffered, straight
// from HBM/L2 with global_load_lds), exactly as the prefill streams K.
//   1. Screening: S^T = K_gist qbar^T on MFMA with qbar (the mean of the
//      group's query heads, formed in fp32) rounded to bf16.  Each lane owns
//      half the candidates of one row and keeps the KA best by this score in
//      registers: per tile it marks the candidates above its current worst,
//      then replaces the worst once per marked candidate.
//   2. Exact ranking: the two lanes of a row pool their 2 KA survivors, score
//      each against the fp32 qbar (each lane half the dimensions, partner sums
//      exchanged), and take the k best by (score desc, id asc).
// Rounding qbar to bf16 moves a score by a few 1e-4 at these sizes, orders of
// magnitude less than the spacing of the top scores among thousands of
// candidates, so the exact top-k is among the survivors with KA >= k + 4.
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

// (score, id) as one unsigned key ordered like (score desc, id asc): the float
// bits made monotone (negative scores flipped whole, positive ones get the
// sign bit) above ~id.  Scores are never NaN here; -inf maps above 0, so the
// key 0 stands for an empty slot.
__device__ inline unsigned long long make_key(float s, int id) {
  const unsigned u = __float_as_uint(s);
  const unsigned m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)m << 32) | (unsigned)~id;
}
__device__ inline float key_score(unsigned long long k) {
  const unsigned m = (unsigned)(k >> 32);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}
__device__ inline int key_id(unsigned long long k) { return (int)~(unsigned)k; }

template <int D, int KA>
__global__ __launch_bounds__(kThreads, 2) void k_select_prefill(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh, int Hq, int Hkv, int q_begin,
    int q_len, int nqt, float mul, int* __restrict__ sel) {
  using C = SCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned short K0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short K1[kBN * D];
  __shared__ float sc[4][32][64];           // a wave's tile scores: [slot][lane]
  // The exact-ranking epilogue pools 64 ids (in sc) and 64 scores per row: the
  // scores go over the two K tiles when they hold 4 x 32 x 64 floats (d = 128),
  // else into an array of their own.
  constexpr bool kScoresInTiles = 2 * kBN * D * (int)sizeof(unsigned short) >= 4 * 32 * 64 * (int)sizeof(float);
  __shared__ float pool_own[kScoresInTiles ? 1 : 4 * 32 * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int qt = nqt - 1 - (int)blockIdx.x;   // heaviest tiles first
  const int h = blockIdx.y, b = blockIdx.z;
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

  // qbar^T operands, bf16: lane (n, h2) holds d = 8 h2 + 16 ks + 0..7
  bf16x8 qreg[C::KS];
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
      const float inv = 1.f / (float)G;
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(a[2 * e] * inv, a[2 * e + 1] * inv);
      qreg[ks] = __builtin_bit_cast(bf16x8, pk);
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

  // the lane's survivors as 64-bit keys, ascending (key[0] is the worst):
  // high word the order-preserving bits of the score, low word ~id, so a
  // larger key is a better (score desc, id asc) candidate; key 0 is empty
  unsigned long long key[KA];
#pragma unroll
  for (int j = 0; j < KA; ++j) key[j] = 0ull;

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
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], s1, 0, 0, 0);
    }
    // value slot x = 16 half + j is candidate 64 t + 32 half + 8 (j / 4) + 4 h2 + j % 4.
    // The mask marks a superset of the candidates that beat the worst
    // survivor (every candidate while a slot is empty, else score >= the
    // worst's; a NaN score, which ranks as -inf, cannot beat a full set);
    // each marked one is re-checked exactly before it is inserted.
    const float wmin_s = key_score(key[0]);
    const bool fill = key[0] == 0ull || wmin_s == -__builtin_inff();
    unsigned mask = 0;
#pragma unroll
    for (int x = 0; x < 32; ++x) {
      const float v = x < 16 ? s0[x & 15] : s1[x & 15];
      sc[wave][x][lane] = v;
      mask |= (unsigned)(v >= wmin_s) << x;
    }
    if (fill) mask = 0xffffffffu;
    if (!rvalid) mask = 0u;
    const int idb = t * kBN + 4 * h2;
    // one sorted insertion per marked candidate, straight-line in every lane
    auto insert_next = [&]() {
      const bool has = mask != 0u;
      const int x = has ? __builtin_ctz(mask) : 0;
      mask &= mask - 1u;
      const int j = x & 15;
      const int id = idb + 32 * (x >> 4) + 8 * (j >> 2) + (j & 3);
      const unsigned long long c = (has && id < ncand) ? make_key(nan_to_neg_inf(sc[wave][x][lane]), id) : 0ull;
      bool bnext = c > key[0];
#pragma unroll
      for (int e = 0; e < KA - 1; ++e) {
        const bool be = bnext;
        bnext = c > key[e + 1];
        key[e] = bnext ? key[e + 1] : (be ? c : key[e]);
      }
      key[KA - 1] = bnext ? c : key[KA - 1];
    };
    // two per trip (the second is a no-op for a lane with nothing left)
    while (__ballot(mask != 0u)) {
      insert_next();
      insert_next();
    }
  };
  for (int t = 0; t < ntile; t += 2) {
    tile(t, K0, K1);
    if (t + 1 < ntile) tile(t + 1, K1, K0);
  }

  // ---- exact ranking of the 2 KA survivors of each row, pooled in LDS (the
  // tile buffers are free now): ids in sc, exact scores over K0/K1
  __syncthreads();
  int* pool_i = reinterpret_cast<int*>(&sc[wave][0][0]) + n * 64;                       // [32 rows][64]
  float* pool_s;
  if constexpr (kScoresInTiles) {
    static_assert(kBN * D * sizeof(unsigned short) == 2 * 2048 * sizeof(float), "two waves' pools per tile buffer");
    pool_s = reinterpret_cast<float*>(wave < 2 ? (void*)K0 : (void*)K1) + (wave & 1) * 2048 + n * 64;
  } else {
    pool_s = pool_own + wave * 2048 + n * 64;
  }
#pragma unroll
  for (int c = 0; c < KA; ++c) pool_i[h2 * KA + c] = key[c] ? key_id(key[c]) : INT_MAX;
  __builtin_amdgcn_wave_barrier();
  // fp32 qbar over this lane's half of the dimensions, d = (D / 2) h2 + 0 .. D / 2 - 1
  float qb[D / 2];
  {
    const unsigned short* q0 = q + b * qsb + (int64_t)rr * qst + (int64_t)(h * G) * qsh + (D / 2) * h2;
#pragma unroll
    for (int e = 0; e < D / 2; ++e) qb[e] = 0.f;
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int c8 = 0; c8 < D / 16; ++c8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(q0 + (int64_t)g * qsh + 8 * c8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qb[8 * c8 + 2 * e] += lo_bf16(w[e]);
          qb[8 * c8 + 2 * e + 1] += hi_bf16(w[e]);
        }
      }
    }
    const float inv = 1.f / (float)G;
#pragma unroll
    for (int e = 0; e < D / 2; ++e) qb[e] *= inv;
  }
  for (int c = 0; c < 2 * KA; ++c) {
    int id = pool_i[c];
    if (id < 0 || id >= ngist_all) id = INT_MAX;   // only real candidates are gathered
    float part = 0.f;
    if (id != INT_MAX) {
      const unsigned short* krow = kb + (int64_t)pos_of(l, K_GIST, id) * kst + (D / 2) * h2;
#pragma unroll
      for (int c8 = 0; c8 < D / 16; ++c8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(krow + 8 * c8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = fmaf(qb[8 * c8 + 2 * e], lo_bf16(w[e]), part);
          part = fmaf(qb[8 * c8 + 2 * e + 1], hi_bf16(w[e]), part);
        }
      }
    }
    // the partner lane holds the other half of the same dot product
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    const float other = __uint_as_float(h2 ? sw[0] : sw[1]);
    if (h2 == 0) {
      pool_s[c] = id != INT_MAX ? nan_to_neg_inf((part + other) * mul) : -__builtin_inff();
      pool_i[c] = id;
    }
  }
  __builtin_amdgcn_wave_barrier();
  // the k best by repeated extraction (lane h2 = 0 of each row), then the
  // chosen ids written at their rank among themselves (ascending)
  if (rvalid && h2 == 0) {
    unsigned long long taken = 0ull;
    int nchosen = 0;
    for (int t = 0; t < l.k; ++t) {
      float bs = -__builtin_inff();
      int bi = INT_MAX, bc = -1;
      for (int c = 0; c < 2 * KA; ++c) {
        const int id = pool_i[c];
        const float sv = pool_s[c];
        if (id != INT_MAX && !((taken >> c) & 1ull) && better(sv, id, bs, bi)) {
          bs = sv;
          bi = id;
          bc = c;
        }
      }
      if (bc < 0) break;
      taken |= 1ull << bc;
      ++nchosen;
    }
    int* out = sel + (((size_t)b * Hkv + h) * q_len + r) * l.k;
    for (int c = 0; c < 2 * KA; ++c) {
      if ((taken >> c) & 1ull) {
        const int id = pool_i[c];
        int rank = 0;
        for (int u = 0; u < 2 * KA; ++u) rank += (((taken >> u) & 1ull) && pool_i[u] < id) ? 1 : 0;
        out[rank] = id;
      }
    }
    for (int t = nchosen; t < l.k; ++t) out[t] = -1;
  }
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
  if (l.k < 1 || l.k > 28) return fail(GSA_EUNSUPPORTED, "top_k %d outside [1, 28]", l.k);
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k", k, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k.dtype != GSA_BF16) return fail(GSA_EUNSUPPORTED, "gsa_select_prefill takes bf16");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (d != 128 && d != 64) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (q_len == 0) return GSA_OK;
  const int nqt = (q_len + kBM - 1) / kBM;
  const float mul = scale / (float)l.g;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(nqt, Hkv, B);
#define GSA_SEL(D, KA)                                                                                      \
  hipLaunchKernelGGL((k_select_prefill<D, KA>), grid, dim3(kThreads), 0, s, l, (const unsigned short*)q.ptr, \
                     q.stride_b, q.stride_t, q.stride_h, (const unsigned short*)k.ptr, k.stride_b, k.stride_t,  \
                     k.stride_h, Hq, Hkv, q_begin, q_len, nqt, mul, sel)
  if (d == 128) {
    if (l.k <= 12) GSA_SEL(128, 16);
    else if (l.k <= 16) GSA_SEL(128, 20);
    else GSA_SEL(128, 32);
  } else {
    if (l.k <= 12) GSA_SEL(64, 16);
    else if (l.k <= 16) GSA_SEL(64, 20);
    else GSA_SEL(64, 32);
  }
#undef GSA_SEL
  return launch_status("gsa_select_prefill");
}
