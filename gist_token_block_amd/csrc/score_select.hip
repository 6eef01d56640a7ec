// Gist scoring and per-KV-group top-k selection (gsa_score_select).
//
// A query scores the chunks whose gists all precede it against their gist
// keys only, and keeps the k best for unfolding (Simplified Sparse Attention
// via Gist Tokens, abstract); with two levels it first keeps the best groups by
// their level-2 gists and then the best chunks inside those groups (Forget,
// Then Recall ... Gist Sparse Attention, abstract).  Score of a candidate for a
// KV head = mean over the KV group's query heads, and over the candidate's
// gists, of q.k * scale; the query-head mean is taken first (qbar), which is
// the same number by linearity.  Order: score descending, then id ascending.
//
// One workgroup per (batch, KV head, query row), with one wave per 64
// candidates up to 16 waves, so every gist key of the row is in flight at
// once.  Lanes of a row group read one key row with 16-byte loads.  Each wave
// keeps a running best-64 list across lanes, merging every scored batch with a
// 64-lane bitonic network (sort the batch, take the element-wise better of
// the running list and the reversed batch, then a bitonic merge).  The waves'
// lists then meet in LDS in a log-depth merge tree.
#include <float.h>
#include <limits.h>

#include "gsa_internal.h"
#include "select_net.h"

namespace gsa {
namespace {

constexpr int kMaxWaves = 16;

template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static void unpack(const u32x4 w, float* out) {
    out[0] = __uint_as_float(w[0]); out[1] = __uint_as_float(w[1]);
    out[2] = __uint_as_float(w[2]); out[3] = __uint_as_float(w[3]);
  }
  __device__ static void load(const float* p, float* out) {
    unpack(*reinterpret_cast<const u32x4*>(p), out);
  }
  __device__ static float one(const float* p) { return *p; }
};
template <> struct Vec16<unsigned short> {
  static constexpr int n = 8;
  __device__ static void unpack(const u32x4 w, float* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = lo_bf16(w[j]);
      out[2 * j + 1] = hi_bf16(w[j]);
    }
  }
  __device__ static void load(const unsigned short* p, float* out) {
    unpack(*reinterpret_cast<const u32x4*>(p), out);
  }
  __device__ static float one(const unsigned short* p) { return bf16_to_f32(*p); }
};

// Candidate -> gist positions / id, for the three kinds of candidate.
struct ChunkCands {        // single level: chunk e, gists pos_of(GIST, e*g + t)
  const Lay* l;
  __device__ int ngist() const { return l->g; }
  __device__ int pos(int e, int t) const { return pos_of(*l, K_GIST, e * l->g + t); }
  __device__ int id(int e) const { return e; }
};
struct GroupCands {        // two levels, level 2: group e
  const Lay* l;
  __device__ int ngist() const { return l->g2; }
  __device__ int pos(int e, int t) const { return pos_of(*l, K_GIST2, e * l->g2 + t); }
  __device__ int id(int e) const { return e; }
};
struct InGroupCands {      // two levels, level 1: chunks of the kept groups
  const Lay* l;
  const int* groups;       // LDS, ascending
  int ngroups;              // groups complete before the query (ids are clamped into range)
  __device__ int chunk(int e) const {
    return iclamp(groups[e / l->G2], 0, ngroups - 1) * l->G2 + e % l->G2;
  }
  __device__ int ngist() const { return l->g; }
  __device__ int pos(int e, int t) const { return pos_of(*l, K_GIST, chunk(e) * l->g + t); }
  __device__ int id(int e) const { return chunk(e); }
};

// Score `ncand` candidates and leave the merged best-64 list in the lanes of
// wave 0 (rs, ri); every wave returns after the block-wide merge.
template <typename T, int D, typename Cands>
__device__ void score_and_rank(const T* __restrict__ kb, int64_t kst, const float* __restrict__ qbar,
                               int ncand, float mul, const Cands& cands, float* __restrict__ score_out,
                               float* lds_s, int* lds_i, float& rs, int& ri) {
  using V = Vec16<T>;
  constexpr int EPL = V::n;          // elements per 16-byte load
  constexpr int LPR = D / EPL;       // lanes per key row
  constexpr int RPI = 64 / LPR;      // key rows per wave instruction
  constexpr int ITER = LPR;          // instructions per batch of 64 rows
  const int lane = __lane_id(), wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int sub = lane % LPR, grp = lane / LPR;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qbar[sub * EPL + e];

  rs = -__builtin_inff();
  ri = INT_MAX;
  const int nbatch = (ncand + 63) / 64;
  const int ng = cands.ngist();
  bool empty = true;   // running list still all -inf: the first sorted batch becomes it
  for (int bi = wave; bi < nbatch; bi += nw) {
    float part[ITER];
    if (ITER <= 16 && ng == 1) {
      // one gist per candidate: issue every row load of the batch, then reduce
      constexpr int NB = ITER <= 16 ? ITER : 1;   // (f32 with d = 128 takes the loop below)
      u32x4 raw[NB];
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        const int e = imin(bi * 64 + grp + RPI * it, ncand - 1);
        raw[it] = *reinterpret_cast<const u32x4*>(kb + (int64_t)cands.pos(e, 0) * kst + sub * EPL);
      }
#pragma unroll
      for (int it = 0; it < NB; ++it) {
        float kv[EPL];
        V::unpack(raw[it], kv);
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) acc = fmaf(qv[x], kv[x], acc);
        part[it] = acc;
      }
    } else {
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int e = bi * 64 + grp + RPI * it;
        float acc = 0.f;
        if (e < ncand) {
          for (int t = 0; t < ng; ++t) {
            float kv[EPL];
            V::load(kb + (int64_t)cands.pos(e, t) * kst + sub * EPL, kv);
#pragma unroll
            for (int x = 0; x < EPL; ++x) acc = fmaf(qv[x], kv[x], acc);
          }
        }
        part[it] = acc;
      }
    }
    float mine = 0.f;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      float v = part[it];
#pragma unroll
      for (int j = 1; j < LPR; j <<= 1) v += xor_lane(v, j);
      if (sub == it) mine = v;
    }
    const int e = bi * 64 + grp + RPI * sub;
    float s = -__builtin_inff();
    int id = INT_MAX;
    if (e < ncand) {
      s = mine * mul;
      id = cands.id(e);
      if (score_out) score_out[id] = s;
      s = nan_to_neg_inf(s);   // a NaN key or query ranks last
    }
    wave_sort_best_first(s, id);
    if (empty) {
      rs = s;
      ri = id;
      empty = false;
    } else {
      wave_merge(rs, ri, s, id);
    }
  }
  // merge tree: at step st, wave w (w % 2st == 0) absorbs wave w + st
  lds_s[wave * 64 + lane] = rs;
  lds_i[wave * 64 + lane] = ri;
  __syncthreads();
  for (int st = 1; st < nw; st <<= 1) {
    if ((wave & (2 * st - 1)) == 0 && wave + st < nw) {
      wave_merge(rs, ri, lds_s[(wave + st) * 64 + lane], lds_i[(wave + st) * 64 + lane]);
      lds_s[wave * 64 + lane] = rs;
      lds_i[wave * 64 + lane] = ri;
    }
    __syncthreads();
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kMaxWaves) void k_score_select(
    Lay l, const T* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh, const T* __restrict__ k,
    int64_t ksb, int64_t kst, int64_t ksh, int Hq, int Hkv, int q_begin, int q_len, float scale,
    int* __restrict__ sel, int* __restrict__ selg, float* __restrict__ scores, int ncols) {
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = Hq / Hkv;
  const int i = q_begin + r;
  const int nthr = blockDim.x;
  __shared__ float qbar[D];
  __shared__ float lds_s[kMaxWaves * 64];
  __shared__ int lds_i[kMaxWaves * 64];
  __shared__ int kept[64];

  for (int e = tid; e < D; e += nthr) {
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += Vec16<T>::one(q + b * qsb + r * qst + (int64_t)(h * G + g) * qsh + e);
    qbar[e] = s / (float)G;
  }
  __syncthreads();
  const T* kb = k + b * ksb + h * ksh;
  const size_t row = ((size_t)b * Hkv + h) * q_len + r;
  float rs;
  int ri;

  if (l.G2 == 0) {
    const int ncand = i >= l.S ? (i - l.S) / l.P : 0;
    float* so = scores ? scores + row * ncols : nullptr;
    if (so)
      for (int e = ncand + tid; e < ncols; e += nthr) so[e] = -__builtin_inff();
    ChunkCands cands{&l};
    score_and_rank<T, D>(kb, kst, qbar, ncand, scale / (float)l.g, cands, so, lds_s, lds_i, rs, ri);
    if (wave == 0) place_ascending(lane < l.k ? ri : INT_MAX, l.k, sel + row * l.k, nullptr);
    return;
  }

  // level 2: groups whose level-2 gists all precede the query
  const int ng2 = i >= l.S ? (i - l.S) / l.P2 : 0;
  float* so = scores ? scores + row * ncols : nullptr;
  if (so)
    for (int e = ng2 + tid; e < ncols; e += nthr) so[e] = -__builtin_inff();
  GroupCands gc{&l};
  score_and_rank<T, D>(kb, kst, qbar, ng2, scale / (float)l.g2, gc, so, lds_s, lds_i, rs, ri);
  __shared__ int nkept;
  if (wave == 0) {
    const int nv = place_ascending(lane < l.k2 ? ri : INT_MAX, l.k2, selg + row * l.k2, kept);
    if (lane == 0) nkept = nv;
  }
  __syncthreads();
  // level 1: chunks of the kept groups
  InGroupCands ic{&l, kept, imax(ng2, 1)};
  score_and_rank<T, D>(kb, kst, qbar, nkept * l.G2, scale / (float)l.g, ic, nullptr, lds_s, lds_i, rs, ri);
  if (wave == 0) place_ascending(lane < l.k ? ri : INT_MAX, l.k, sel + row * l.k, nullptr);
}

template <typename T, int D>
void launch(const Lay& l, const gsa_tensor& q, const gsa_tensor& k, int B, int Hq, int Hkv, int q_begin,
            int q_len, float scale, int* sel, int* selg, float* scores, int ncols, hipStream_t st) {
  // one wave per 64 candidates of the busiest row (either level), 1..16 waves
  const int i_max = q_begin + q_len - 1;
  int nmax = l.G2 == 0 ? (i_max >= l.S ? (i_max - l.S) / l.P : 0)
                       : imax(i_max >= l.S ? (i_max - l.S) / l.P2 : 0, l.k2 * l.G2);
  const int waves = iclamp((nmax + 63) / 64, 1, kMaxWaves);
  hipLaunchKernelGGL((k_score_select<T, D>), dim3(q_len, Hkv, B), dim3(64 * waves), 0, st, l,
                     (const T*)q.ptr, q.stride_b, q.stride_t, q.stride_h, (const T*)k.ptr, k.stride_b,
                     k.stride_t, k.stride_h, Hq, Hkv, q_begin, q_len, scale, sel, selg, scores, ncols);
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status gsa_score_select(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, int32_t B,
                                       int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                                       int32_t q_begin, int32_t q_len, float scale, int32_t* sel,
                                       int32_t* sel_groups, float* scores, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, 64, &l);
  if (st != GSA_OK) return st;
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k", k, d)) != GSA_OK) return st;
  if (q.dtype != k.dtype) return fail(GSA_EINVAL, "q and k dtypes differ");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (l.k < 1 || l.k > 64) return fail(GSA_EUNSUPPORTED, "top_k %d outside [1, 64]", l.k);
  if (l.G2 > 0 && l.k2 > 64) return fail(GSA_EUNSUPPORTED, "l2_top_k %d > 64", l.k2);
  if (l.G2 > 0 && l.k2 * l.G2 > 1 << 20) return fail(GSA_EUNSUPPORTED, "l2_top_k * l2_chunks too large");
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is NULL with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  const int ncols = gsa_score_columns(layout, seq_len);
  hipStream_t s = (hipStream_t)stream;
  if (q.dtype == GSA_F32) {
    if (d == 64) launch<float, 64>(l, q, k, B, Hq, Hkv, q_begin, q_len, scale, sel, sel_groups, scores, ncols, s);
    else launch<float, 128>(l, q, k, B, Hq, Hkv, q_begin, q_len, scale, sel, sel_groups, scores, ncols, s);
  } else {
    if (d == 64) launch<unsigned short, 64>(l, q, k, B, Hq, Hkv, q_begin, q_len, scale, sel, sel_groups, scores, ncols, s);
    else launch<unsigned short, 128>(l, q, k, B, Hq, Hkv, q_begin, q_len, scale, sel, sel_groups, scores, ncols, s);
  }
  return launch_status("gsa_score_select");
}
