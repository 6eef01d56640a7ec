// Backward of the prefill with selective unfolding, for the unfolded keys.
//
// The forward (gsa_attn_prefill_unfolded) attends each query to a fixed part
// (sinks, earlier gists, its window) and to the raw tokens of its chosen
// chunks before the window (Simplified Sparse Attention via Gist Tokens,
// abstract: unfold the top-k chunks; Forget, Then Recall ... Gist Sparse
// Attention, abstract: the pattern is trained end to end).  The two key sets
// are disjoint, so the gradients split the same way: the fixed part's run on
// the fixed layout's tables (backward.hip), and the kernels here add the
// unfolded keys' share, with P recomputed from the forward's log-sum-exp over
// the union and D = rowsum(dO * O) from the fixed part's first kernel:
//   k_unfold_bwd_q   one wave per (batch, KV head, query row): gathers the
//                    row's unfolded K and V rows and adds scale dS K to dq;
//   k_unfold_bwd_kv  one wave per (batch, KV head, chunk): walks the query
//                    rows that unfolded the chunk (a per-chunk list built by
//                    count, scan and fill, sorted in the wave so the sums run
//                    in a fixed order) and adds scale dS^T Q and P^T dO to the
//                    chunk's raw rows of dk and dv.
#include <limits.h>

#include "gsa_internal.h"
#include "select_net.h"

namespace gsa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxKeys = 64;    // unfolded raws per pass of a wave
constexpr int kMaxG = 16;
constexpr int kMaxC = 16;       // raws per chunk the chunk kernel holds
constexpr int kSortCap = 1024;  // selecting rows of a chunk sorted in LDS (more: list order)

template <typename T> struct GradIO;
template <> struct GradIO<float> {
  __device__ static float get(const float* p) { return *p; }
  __device__ static void put(float* p, float x) { *p = x; }
};
template <> struct GradIO<unsigned short> {
  __device__ static float get(const unsigned short* p) { return bf16_to_f32(*p); }
  __device__ static void put(unsigned short* p, float x) { *p = (unsigned short)(pack_bf16x2(x, 0.f) & 0xffffu); }
};

// The unfolded raws of one query row: lane e < k holds chosen chunk e's first
// raw position and how many of its raws lie before the window; nk = total.
struct UnfoldRow {
  int st, len, excl, nk;
};
__device__ inline UnfoldRow unfold_row(const Lay& l, const int* sel_row, int i, int lane) {
  const int lo = imax(0, i - l.W1 + 1);
  const int nch = count_below(l, K_GIST, i) / l.g;   // complete chunks
  int len = 0, st = 0;
  if (lane < l.k) {
    const int m = sel_row[lane];
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
  UnfoldRow u;
  u.st = st;
  u.len = len;
  u.excl = incl - len;
  u.nk = __shfl(incl, 63);
  return u;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) v += xor_lane(v, j);
  return v;
}

// ------------------------------------------------------------------ dQ
template <int D, int MG, typename TG>
__global__ __launch_bounds__(64 * kWaves) void k_unfold_bwd_q(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh,
    const unsigned short* __restrict__ dO, int64_t dsb, int64_t dst, int64_t dsh,
    const float* __restrict__ lse2, const float* __restrict__ delta, TG* __restrict__ dq, int64_t gsb, int64_t gst,
    int64_t gsh, int B, int Hq, int Hkv, int q_begin, int q_len, const int* __restrict__ sel, float c2,
    float scale) {
  constexpr int DPL = D / 64;   // dq dimensions per lane
  __shared__ float qs[kWaves][MG][D];
  __shared__ float os[kWaves][MG][D];
  __shared__ float dss[kWaves][MG][kMaxKeys];
  __shared__ int kpos[kWaves][kMaxKeys];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = Hq / Hkv;
  const long long total = (long long)B * Hkv * q_len;
  for (long long item = (long long)blockIdx.x * kWaves + wave; item < total; item += (long long)gridDim.x * kWaves) {
    const int r = (int)(item % q_len);
    const int h = (int)((item / q_len) % Hkv);
    const int b = (int)(item / ((long long)q_len * Hkv));
    const int i = q_begin + r;
    const UnfoldRow u = unfold_row(l, sel + (((size_t)b * Hkv + h) * q_len + r) * l.k, i, lane);
    if (u.nk == 0) continue;   // wave-uniform
    for (int x = lane; x < G * D; x += 64) {
      const int hd = x / D, dd = x - hd * D;
      qs[wave][hd][dd] = bf16_to_f32(q[b * qsb + (int64_t)r * qst + (int64_t)(h * G + hd) * qsh + dd]);
      os[wave][hd][dd] = bf16_to_f32(dO[b * dsb + (int64_t)r * dst + (int64_t)(h * G + hd) * dsh + dd]);
    }
    float l2[MG], dl[MG], acc[MG][DPL];
#pragma unroll
    for (int hd = 0; hd < MG; ++hd) {
      const size_t ri = ((size_t)b * Hq + h * G + imin(hd, G - 1)) * q_len + r;
      l2[hd] = lse2[ri];
      dl[hd] = delta[ri];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hd][e] = 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    for (int k0 = 0; k0 < u.nk; k0 += kMaxKeys) {
      // position of unfolded key k0 + lane: the run (chunk) holding it
      int p = -1;
      const int kk = k0 + lane;
      for (int e = 0; e < l.k && e < 64; ++e) {
        const int s_e = __shfl(u.excl, e), l_e = __shfl(u.len, e), st_e = __shfl(u.st, e);
        if (kk >= s_e && kk < s_e + l_e) p = st_e + (kk - s_e);
      }
      kpos[wave][lane] = p;
      // logits and dP of key lane for every head: K row, then V row, each
      // loaded whole before its dot products
      float lg[MG], dp[MG];
#pragma unroll
      for (int hd = 0; hd < MG; ++hd) lg[hd] = dp[hd] = 0.f;
      {
        u32x4 w[D / 8];
        const unsigned short* krow = k + b * ksb + (int64_t)imax(p, 0) * kst + h * ksh;
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8)
          w[c8] = p >= 0 ? *reinterpret_cast<const u32x4*>(krow + 8 * c8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int hd = 0; hd < MG; ++hd) {
          if (hd < G) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                a0 = fmaf(qs[wave][hd][8 * c8 + 2 * e], lo_bf16(w[c8][e]), a0);
                a1 = fmaf(qs[wave][hd][8 * c8 + 2 * e + 1], hi_bf16(w[c8][e]), a1);
              }
            }
            lg[hd] = a0 + a1;
          }
        }
        const unsigned short* vrow = v + b * vsb + (int64_t)imax(p, 0) * vst + h * vsh;
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8)
          w[c8] = p >= 0 ? *reinterpret_cast<const u32x4*>(vrow + 8 * c8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int hd = 0; hd < MG; ++hd) {
          if (hd < G) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c8 = 0; c8 < D / 8; ++c8) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                a0 = fmaf(os[wave][hd][8 * c8 + 2 * e], lo_bf16(w[c8][e]), a0);
                a1 = fmaf(os[wave][hd][8 * c8 + 2 * e + 1], hi_bf16(w[c8][e]), a1);
              }
            }
            dp[hd] = a0 + a1;
          }
        }
      }
      // dS = P (dP - D), P from the forward's log-sum-exp (base 2)
#pragma unroll
      for (int hd = 0; hd < MG; ++hd) {
        if (hd < G) {
          const float pr = p >= 0 ? __builtin_amdgcn_exp2f(fmaf(lg[hd], c2, -l2[hd])) : 0.f;
          dss[wave][hd][lane] = pr * (dp[hd] - dl[hd]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // dq += dS K: lane owns dimensions lane * DPL .. + DPL - 1; every K load
      // of the pass is issued before the products
      const int nkp = imin(kMaxKeys, u.nk - k0);
      unsigned kw[kMaxKeys];
#pragma unroll
      for (int j = 0; j < kMaxKeys; ++j) {
        kw[j] = 0u;
        if (j < nkp) {
          const int pj = kpos[wave][j];
          const unsigned short* kr = k + b * ksb + (int64_t)pj * kst + h * ksh + lane * DPL;
          if constexpr (DPL == 2) kw[j] = *reinterpret_cast<const unsigned*>(kr);
          else kw[j] = (unsigned)kr[0] << 16;
        }
      }
#pragma unroll
      for (int j4 = 0; j4 < kMaxKeys; j4 += 4) {
        if (j4 < nkp) {
#pragma unroll
          for (int hd = 0; hd < MG; ++hd) {
            if (hd < G) {
              const f32x4 ds4 = *reinterpret_cast<const f32x4*>(&dss[wave][hd][j4]);
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                if constexpr (DPL == 2) {
                  acc[hd][0] = fmaf(ds4[jj], lo_bf16(kw[j4 + jj]), acc[hd][0]);
                  acc[hd][1] = fmaf(ds4[jj], hi_bf16(kw[j4 + jj]), acc[hd][1]);
                } else {
                  acc[hd][0] = fmaf(ds4[jj], hi_bf16(kw[j4 + jj]), acc[hd][0]);
                }
              }
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // add to the fixed part's dq
#pragma unroll
    for (int hd = 0; hd < MG; ++hd) {
      if (hd < G) {
        TG* row = dq + b * gsb + (int64_t)r * gst + (int64_t)(h * G + hd) * gsh + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) GradIO<TG>::put(row + e, GradIO<TG>::get(row + e) + scale * acc[hd][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------------ per-chunk lists
// Entry (row r, choice e) counts for chunk m when some of m's raws lie before
// r's window (the raws the forward unfolded for r).
__device__ inline int unfolded_chunk(const Lay& l, const int* sel, int b, int h, int Hkv, int q_len, int q_begin,
                                     int r, int e) {
  const int m = sel[(((size_t)b * Hkv + h) * q_len + r) * l.k + e];
  const int i = q_begin + r;
  const int nch = count_below(l, K_GIST, i) / l.g;
  if (m < 0 || m >= nch) return -1;
  const int lo = imax(0, i - l.W1 + 1);
  return pos_of(l, K_RAW, m * l.c) < lo ? m : -1;
}

__global__ void k_fill_zero(int* __restrict__ p, long long n) {
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long long)gridDim.x * blockDim.x)
    p[x] = 0;
}

__global__ void k_chunk_count(Lay l, const int* __restrict__ sel, int B, int Hkv, int q_begin, int q_len, int nch,
                              int* __restrict__ cnt) {
  const long long total = (long long)B * Hkv * q_len * l.k;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < total; x += (long long)gridDim.x * blockDim.x) {
    const int e = (int)(x % l.k);
    const long long y = x / l.k;
    const int r = (int)(y % q_len);
    const int h = (int)((y / q_len) % Hkv);
    const int b = (int)(y / ((long long)q_len * Hkv));
    const int m = unfolded_chunk(l, sel, b, h, Hkv, q_len, q_begin, r, e);
    if (m >= 0) atomicAdd(&cnt[((size_t)b * Hkv + h) * nch + m], 1);
  }
}

// Exclusive scan of one group's counts (one workgroup per (batch, KV head)):
// off[g][m], m = 0 .. nch (off[g][nch] = the group's entries).
__global__ __launch_bounds__(256) void k_chunk_scan(const int* __restrict__ cnt, int* __restrict__ off, int nch) {
  __shared__ int part[256];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int per = (nch + 255) / 256;
  const int m0 = imin(tid * per, nch), m1 = imin(m0 + per, nch);
  const int* c = cnt + (size_t)g * nch;
  int s = 0;
  for (int m = m0; m < m1; ++m) s += c[m];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {   // inclusive scan of the 256 partial sums
    const int t = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += t;
    __syncthreads();
  }
  int run = part[tid] - s;
  int* o = off + (size_t)g * (nch + 1);
  for (int m = m0; m < m1; ++m) {
    o[m] = run;
    run += c[m];
  }
  if (tid == 255) o[nch] = part[255];
}

__global__ void k_chunk_fill(Lay l, const int* __restrict__ sel, int B, int Hkv, int q_begin, int q_len, int nch,
                             const int* __restrict__ off, int* __restrict__ cursor, int* __restrict__ list) {
  const long long total = (long long)B * Hkv * q_len * l.k;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < total; x += (long long)gridDim.x * blockDim.x) {
    const int e = (int)(x % l.k);
    const long long y = x / l.k;
    const int r = (int)(y % q_len);
    const int h = (int)((y / q_len) % Hkv);
    const int b = (int)(y / ((long long)q_len * Hkv));
    const int m = unfolded_chunk(l, sel, b, h, Hkv, q_len, q_begin, r, e);
    if (m >= 0) {
      const size_t g = (size_t)b * Hkv + h;
      const int slot = atomicAdd(&cursor[g * nch + m], 1);
      list[g * (size_t)q_len * l.k + off[g * (nch + 1) + m] + slot] = r;
    }
  }
}

// ------------------------------------------------------------------ dK, dV
// CM (a power of two, 2 .. 16) bounds the raws per chunk.  Lane layout: the
// wave holds S = 2048 / (D CM) (row, query head) pairs at once, one per slot
// of LS = 64 / S lanes; a lane owns DL = 32 / CM dimensions of its slot's
// pair and of every raw of the chunk, so each load fetches distinct bytes and
// one q or dO load instruction covers S pairs.  Logits and dP are packed bf16
// dot products summed over the slot's lanes; each lane accumulates its
// dimensions of dK and dV for every raw, and the slots' sums are added at the
// end.  Pairs go in batches of KP steps: the lanes of a slot look up the
// rows, heads, log-sum-exps and D of the batch's pairs, and every q and dO
// load of the batch is issued, packed, before the first product.

template <int N> __device__ inline void load_words(const unsigned short* p, unsigned (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(p + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * c + e] = x[e];
    }
  } else if constexpr (N == 2) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    w[0] = x[0];
    w[1] = x[1];
  } else {
    static_assert(N == 1, "1, 2 or a multiple of 4 words");
    w[0] = *reinterpret_cast<const unsigned*>(p);
  }
}

template <int CTRL> __device__ inline float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the LS lanes of a slot (aligned groups of LS lanes), in every lane.
template <int LS> __device__ inline float slot_sum(float v) {
  if constexpr (LS >= 16) {
    v = dpp_add<0x128>(v);   // row_ror:8 (rotations within a 16-lane row reduce it in 4 steps)
    v = dpp_add<0x124>(v);   // row_ror:4
    v = dpp_add<0x122>(v);   // row_ror:2
    v = dpp_add<0x121>(v);   // row_ror:1
    if constexpr (LS >= 32) v += xor_lane(v, 16);
    if constexpr (LS >= 64) v += xor_lane(v, 32);
  } else if constexpr (LS == 8) {
    v = dpp_add<0x141>(v);   // row_half_mirror: lane i + lane 7 - i
    v = dpp_add<0xB1>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E>(v);    // quad_perm [2,3,0,1]
  } else if constexpr (LS == 4) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
  } else {
    static_assert(LS == 2, "slots of 2 .. 64 lanes");
    v = dpp_add<0xB1>(v);
  }
  return v;
}

// Sum over the slots of the lanes at the same place in each slot.
template <int LS> __device__ inline float cross_slot_sum(float v) {
  if constexpr (LS <= 8) v = dpp_add<0x128>(v);   // row_ror:8
  if constexpr (LS <= 4) v = dpp_add<0x124>(v);   // row_ror:4
  if constexpr (LS <= 2) v = dpp_add<0x122>(v);   // row_ror:2
  if constexpr (LS <= 16) v += xor_lane(v, 16);
  if constexpr (LS <= 32) v += xor_lane(v, 32);
  return v;
}

template <int D, int CM, typename TG>
__global__ __launch_bounds__(64 * kWaves) void k_unfold_bwd_kv(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh,
    const unsigned short* __restrict__ dO, int64_t dsb, int64_t dst, int64_t dsh,
    const float* __restrict__ lse2, const float* __restrict__ delta, TG* __restrict__ dk, int64_t ksb_o,
    int64_t kst_o, int64_t ksh_o, TG* __restrict__ dv, int64_t vsb_o, int64_t vst_o, int64_t vsh_o, int B, int Hq,
    int Hkv, int q_begin, int q_len, int nch, const int* __restrict__ off, const int* __restrict__ list, float c2,
    float scale) {
  constexpr int DL = 32 / CM;                 // dimensions per lane
  constexpr int NW = DL / 2;                  // packed bf16 words per lane and row
  constexpr int LS = D / DL;                  // lanes per slot
  constexpr int S = 64 / LS;                  // pairs per step
  constexpr int KP = LS < 8 ? LS : (DL > 8 ? 4 : 8);   // steps per batch (at most LS: one lookup lane each)
  static_assert(LS * S == 64 && LS >= 2, "D * CM between 128 and 2048");
  __shared__ int seg[kWaves][kSortCap];
  __shared__ int srt[kWaves][kSortCap];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LS, sl = lane % LS, d0 = DL * sl;
  const int G = Hq / Hkv;
  const int C = imin(l.c, CM);
  const long long total = (long long)B * Hkv * nch;
  for (long long item = (long long)blockIdx.x * kWaves + wave; item < total; item += (long long)gridDim.x * kWaves) {
    const int m = (int)(item % nch);
    const int h = (int)((item / nch) % Hkv);
    const int b = (int)(item / ((long long)nch * Hkv));
    const size_t g = (size_t)b * Hkv + h;
    const int o0 = off[g * (nch + 1) + m], n = off[g * (nch + 1) + m + 1] - o0;
    if (n <= 0) continue;   // wave-uniform
    const int* rows = list + g * (size_t)q_len * l.k + o0;
    // the rows in ascending order: each entry's place is its rank (ties,
    // which a valid selection never has, go by list position)
    const bool sorted = n <= kSortCap;
    if (sorted) {
      for (int x = lane; x < n; x += 64) seg[wave][x] = rows[x];
      __builtin_amdgcn_wave_barrier();
      for (int x = lane; x < n; x += 64) {
        const int rv = seg[wave][x];
        int rank = 0;
        for (int y = 0; y < n; ++y) {
          const int sv = seg[wave][y];
          rank += (sv < rv || (sv == rv && y < x)) ? 1 : 0;
        }
        srt[wave][rank] = rv;
      }
      __builtin_amdgcn_wave_barrier();
    }
    const int st = pos_of(l, K_RAW, m * l.c);
    // this lane's dimensions of every raw of the chunk (raws past its end
    // re-read the last one; their P is 0)
    unsigned kw[CM][NW], vw[CM][NW];
#pragma unroll
    for (int t = 0; t < CM; ++t) {
      const int row = st + imin(t, C - 1);
      load_words<NW>(k + b * ksb + (int64_t)row * kst + h * ksh + d0, kw[t]);
      load_words<NW>(v + b * vsb + (int64_t)row * vst + h * vsh + d0, vw[t]);
    }
    float gk[CM][DL], gv[CM][DL];
#pragma unroll
    for (int t = 0; t < CM; ++t)
#pragma unroll
      for (int e = 0; e < DL; ++e) gk[t][e] = gv[t][e] = 0.f;
    const int npair = n * G;
    const int64_t qb = b * qsb + (int64_t)h * G * qsh + d0, ob = b * dsb + (int64_t)h * G * dsh + d0;
    for (int p0 = 0; p0 < npair; p0 += KP * S) {
      // lane sl < KP of each slot: pair p0 + sl S + slot (row * 16 + head, -1 past the end)
      int rh = -1;
      float l2v = 0.f, dlv = 0.f;
      if (sl < KP) {
        const int pid = p0 + sl * S + slot;
        if (pid < npair) {
          const int x = pid / G, hd = pid - x * G;
          const int r = sorted ? srt[wave][x] : rows[x];
          rh = r * 16 + hd;
          const size_t ri = ((size_t)b * Hq + h * G + hd) * q_len + r;
          l2v = lse2[ri];
          dlv = delta[ri];
        }
      }
      unsigned qw[KP][NW], ow[KP][NW];
      int rhj[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        rhj[j] = __shfl(rh, slot * LS + j);
        const int x = imax(rhj[j], 0), r = x >> 4, hd = x & 15;
        load_words<NW>(q + qb + (int64_t)r * qst + (int64_t)hd * qsh, qw[j]);
        load_words<NW>(dO + ob + (int64_t)r * dst + (int64_t)hd * dsh, ow[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const float l2 = __shfl(l2v, slot * LS + j), dl = __shfl(dlv, slot * LS + j);
        float sc[CM], dp[CM];
#pragma unroll
        for (int t = 0; t < CM; ++t) {
          float a = 0.f, c = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[j][w]),
                                                __builtin_bit_cast(bf16x2, kw[t][w]), a, false);
            c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ow[j][w]),
                                                __builtin_bit_cast(bf16x2, vw[t][w]), c, false);
          }
          sc[t] = slot_sum<LS>(a);
          dp[t] = slot_sum<LS>(c);
        }
        float qf[DL], of[DL];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          qf[2 * w] = lo_bf16(qw[j][w]);
          qf[2 * w + 1] = hi_bf16(qw[j][w]);
          of[2 * w] = lo_bf16(ow[j][w]);
          of[2 * w + 1] = hi_bf16(ow[j][w]);
        }
        // raw t lies before the row's window (none for the padding)
        const int lim = rhj[j] >= 0 ? q_begin + (rhj[j] >> 4) - l.W1 + 1 - st : 0;
#pragma unroll
        for (int t = 0; t < CM; ++t) {
          const bool vis = t < C && t < lim;
          const float pr = vis ? __builtin_amdgcn_exp2f(fmaf(sc[t], c2, -l2)) : 0.f;
          const float ds = scale * pr * (dp[t] - dl);
#pragma unroll
          for (int e = 0; e < DL; ++e) {
            gk[t][e] = fmaf(ds, qf[e], gk[t][e]);
            gv[t][e] = fmaf(pr, of[e], gv[t][e]);
          }
        }
      }
    }
    // add the slots' sums to the fixed part's dk and dv; slot s writes the
    // raws t with t mod S = s
#pragma unroll
    for (int t = 0; t < CM; ++t) {
#pragma unroll
      for (int e = 0; e < DL; ++e) {
        gk[t][e] = cross_slot_sum<LS>(gk[t][e]);
        gv[t][e] = cross_slot_sum<LS>(gv[t][e]);
      }
      if (t < C && t % S == slot) {
        TG* kr = dk + b * ksb_o + (int64_t)(st + t) * kst_o + h * ksh_o + d0;
        TG* vr = dv + b * vsb_o + (int64_t)(st + t) * vst_o + h * vsh_o + d0;
#pragma unroll
        for (int e = 0; e < DL; ++e) {
          GradIO<TG>::put(kr + e, GradIO<TG>::get(kr + e) + gk[t][e]);
          GradIO<TG>::put(vr + e, GradIO<TG>::get(vr + e) + gv[t][e]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

// Sizes of the per-chunk lists in the workspace after the fixed part's
// 2 B Hq q_len floats: counts and cursors [B Hkv][nch], offsets
// [B Hkv][nch + 1], rows [B Hkv][q_len k], each 256-byte aligned.
size_t unfold_backward_extra_bytes(const Lay& l, int B, int Hkv, int q_len, int nch) {
  const size_t groups = (size_t)B * Hkv;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * al(groups * nch * sizeof(int)) + al(groups * (nch + 1) * sizeof(int)) +
         al(groups * (size_t)q_len * l.k * sizeof(int));
}

gsa_status launch_unfold_backward(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k, const gsa_tensor& v,
                                  const gsa_tensor& dO, const gsa_tensor& dq, const gsa_tensor& dk,
                                  const gsa_tensor& dv, int B, int Hq, int Hkv, int q_begin, int q_len,
                                  const int* sel, int nch, float scale, const float* lse2, const float* delta,
                                  char* extra, hipStream_t st, int phase) {
  const int G = Hq / Hkv;
  if (G > kMaxG) return fail(GSA_EUNSUPPORTED, "more than %d query heads per KV head", kMaxG);
  if (l.k > 64) return fail(GSA_EUNSUPPORTED, "top_k %d > 64", l.k);
  if (l.c > kMaxC) return fail(GSA_EUNSUPPORTED, "chunk_len %d > %d in the unfolded backward", l.c, kMaxC);
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const float c2 = scale * kLog2e;
  const bool f32 = dq.dtype == GSA_F32;
  if (phase == 0) {   // dq
    const long long items = (long long)B * Hkv * q_len;
    const long long want = (items + kWaves - 1) / kWaves;
    const int grid = (int)(want < 8LL * cus ? want : 8LL * cus);
#define GSA_UQ(D, MG, TG)                                                                                       \
  hipLaunchKernelGGL((k_unfold_bwd_q<D, MG, TG>), dim3(grid), dim3(64 * kWaves), 0, st, l,                     \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h, (const unsigned short*)k.ptr, \
                     k.stride_b, k.stride_t, k.stride_h, (const unsigned short*)v.ptr, v.stride_b, v.stride_t,        \
                     v.stride_h, (const unsigned short*)dO.ptr, dO.stride_b, dO.stride_t, dO.stride_h, lse2, delta,   \
                     (TG*)dq.ptr, dq.stride_b, dq.stride_t, dq.stride_h, B, Hq, Hkv, q_begin, q_len, sel, c2, scale)
#define GSA_UQ2(D, MG)                                 \
  if (f32) GSA_UQ(D, MG, float);                       \
  else GSA_UQ(D, MG, unsigned short)
    if (d == 128) {
      if (G <= 4) GSA_UQ2(128, 4);
      else if (G <= 8) GSA_UQ2(128, 8);
      else GSA_UQ2(128, 16);
    } else {
      if (G <= 4) GSA_UQ2(64, 4);
      else if (G <= 8) GSA_UQ2(64, 8);
      else GSA_UQ2(64, 16);
    }
#undef GSA_UQ2
#undef GSA_UQ
    return launch_status("gsa_attn_prefill_unfolded_backward (dq)");
  }
  // dk, dv: per-chunk lists, then the chunk kernel
  const size_t groups = (size_t)B * Hkv;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  int* cnt = (int*)extra;
  int* cursor = (int*)(extra + al(groups * nch * sizeof(int)));
  int* offs = (int*)(extra + 2 * al(groups * nch * sizeof(int)));
  int* list = (int*)(extra + 2 * al(groups * nch * sizeof(int)) + al(groups * (nch + 1) * sizeof(int)));
  const long long zn = 2LL * (long long)(al(groups * nch * sizeof(int)) / sizeof(int));
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)imin((int)((zn + 255) / 256), 4 * cus)), dim3(256), 0, st, cnt, zn);
  const long long entries = (long long)B * Hkv * q_len * l.k;
  const int egrid = (int)imin((int)((entries + 255) / 256), 8 * cus);
  hipLaunchKernelGGL(k_chunk_count, dim3(egrid), dim3(256), 0, st, l, sel, B, Hkv, q_begin, q_len, nch, cnt);
  hipLaunchKernelGGL(k_chunk_scan, dim3((unsigned)groups), dim3(256), 0, st, cnt, offs, nch);
  hipLaunchKernelGGL(k_chunk_fill, dim3(egrid), dim3(256), 0, st, l, sel, B, Hkv, q_begin, q_len, nch, offs, cursor,
                     list);
  const long long items = (long long)groups * nch;
  const long long want = (items + kWaves - 1) / kWaves;
  const int grid = (int)(want < 8LL * cus ? want : 8LL * cus);
#define GSA_UKV(D, MG, TG)                                                                                         \
  hipLaunchKernelGGL((k_unfold_bwd_kv<D, MG, TG>), dim3(grid), dim3(64 * kWaves), 0, st, l,                        \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h, (const unsigned short*)k.ptr,    \
                     k.stride_b, k.stride_t, k.stride_h, (const unsigned short*)v.ptr, v.stride_b, v.stride_t,           \
                     v.stride_h, (const unsigned short*)dO.ptr, dO.stride_b, dO.stride_t, dO.stride_h, lse2, delta,      \
                     (TG*)dk.ptr, dk.stride_b, dk.stride_t, dk.stride_h, (TG*)dv.ptr, dv.stride_b, dv.stride_t,          \
                     dv.stride_h, B, Hq, Hkv, q_begin, q_len, nch, offs, list, c2, scale)
#define GSA_UKV2(D, CM)                    \
  if (f32) GSA_UKV(D, CM, float);          \
  else GSA_UKV(D, CM, unsigned short)
#define GSA_UKV3(D)                        \
  if (l.c <= 2) GSA_UKV2(D, 2);            \
  else if (l.c <= 4) GSA_UKV2(D, 4);       \
  else if (l.c <= 8) GSA_UKV2(D, 8);       \
  else GSA_UKV2(D, 16)
  if (d == 128) {
    GSA_UKV3(128);
  } else {
    GSA_UKV3(64);
  }
#undef GSA_UKV3
#undef GSA_UKV2
#undef GSA_UKV
  return launch_status("gsa_attn_prefill_unfolded_backward (dk, dv)");
}

}  // namespace gsa
