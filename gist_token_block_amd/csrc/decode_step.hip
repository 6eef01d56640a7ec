// Fused decode step (gsa_decode_step): scoring, per-KV-group top-k (one or two
// levels) and the split-K attention of one query token per sequence, with
// every visible K/V row read from HBM once.
//
// The method: a query scores the chunks whose gists all precede it against
// their gist keys only and unfolds the raw tokens of the k best (Simplified
// Sparse Attention via Gist Tokens, abstract); with gist of gist it first keeps
// the best groups by their level-2 gists, then the best chunks inside them
// (Forget, Then Recall ... Gist Sparse Attention, abstract).  It attends to the
// sinks, every gist (two levels: every level-2 gist and the level-1 gists of
// the kept groups), its local window and the unfolded raws (UniGist summary,
// Approach).  A candidate's score for one KV head is the mean over that KV
// group's query heads (and over the candidate's gists) of q.k * scale.
//
// Every scored gist is also a visible row, so scoring costs no extra reads:
//   phase A (k_step_a, many workgroups per (batch, KV head)): stream the
//     top-level gist stream (single level: the gists; two levels: the level-2
//     gists), the sinks and the window; one MFMA product per 16 rows gives the
//     logits of all query heads, which feed both the attention partial and,
//     summed over the heads, the candidates' scores.  Each workgroup keeps the
//     best k of its candidates.  With two levels the last workgroup of a
//     (batch, KV head) to finish merges those lists into the group selection,
//     streams the kept groups' level-1 gists (scoring and attending them) and
//     picks the chunks.
//   phase B (k_step_b, many workgroups per (batch, KV head)): with one level,
//     every workgroup merges phase A's lists into the selection itself (one
//     load of a few lists, where it would otherwise read the selection), so
//     phase A ends without a completion count; then stream the raw rows of
//     the unfolded chunks; the last workgroup merges the partials of both
//     phases with log-sum-exp weights and writes the output.
// Rows inside the window are attended only by the window segment, so every
// row is counted once; top-level gists inside the window are still scored.
#include <limits.h>

#include "decode_stream.h"

namespace gsa {
namespace {
using namespace dec;

constexpr int kMaxRowsPerSplit = 2048;   // rows one phase-A workgroup scores
constexpr int kMaxL1Rows = 1024;         // level-1 gist rows of the kept groups

struct StepArgs {
  Lay l;
  const unsigned short* q;
  int64_t qsb, qsh;
  const unsigned short* kc;
  int64_t ksb, kst, ksh;
  const unsigned short* vc;
  int64_t vsb, vst, vsh;
  int Hq, Hkv, kv_len;
  float c2, score_mul1, score_mul2;   // logit scale (log2 units); score scales for levels 1 and 2
  int* counters;                      // [2][B*Hkv]: phase A, phase B
  float* list_s;                      // [B*Hkv][nsa][64]
  int* list_i;
  float* part;                        // [B*Hkv][nslot][G][D + kPartExtra]
  int nsa, rpa, nsb, rpb, nslot;
  int* sel;                           // [B*Hkv][k]      (out)
  int* selg;                          // [B*Hkv][k2]     (out, two levels)
  void* o;
  int64_t osb, osh;
  float* lse;
};

template <int D>
__device__ void load_q(const StepArgs& a, int b, int h, bf16x8* qreg) {
  using C = DCfg<D>;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const unsigned short* qrow = a.q + b * a.qsb + (int64_t)(h * G + imin(col, G - 1)) * a.qsh;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * grp + 32 * ks);
    if (col >= G) w = u32x4{0u, 0u, 0u, 0u};
    qreg[ks] = __builtin_bit_cast(bf16x8, w);
  }
}

// ---------------------------------------------------------------- phase A
template <int D>
__global__ __launch_bounds__(kThreads) void k_step_a(StepArgs a) {
  using C = DCfg<D>;
  const Lay& l = a.l;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int i = a.kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);
  const size_t gidx = (size_t)b * a.Hkv + h;
  const bool two = l.G2 > 0;
  const int top = two ? K_GIST2 : K_GIST;            // the stream scored here
  const int per = two ? l.g2 : l.g;                  // its gists per candidate
  const int ktop = two ? l.k2 : l.k;                 // candidates kept
  const int ncand = count_below(l, top, i) / per;    // complete candidates
  const int natt = count_below(l, top, lo);          // top gists before the window
  const int nsc = ncand * per;                       // top gists that are scored
  const int ntop = imax(natt, nsc);
  const int nsink = imin(l.S, lo);
  const int total = ntop + nsink + (i - lo + 1);     // [top | sinks | window]

  __shared__ __attribute__((aligned(1024))) StepLds<D> lds;
  __shared__ int rowpos[2][kRows], rowflag[3][kRows];
  __shared__ float rowscore[kMaxRowsPerSplit];
  __shared__ float lds_s[4 * 64];
  __shared__ int lds_i[4 * 64];
  __shared__ float wstat[192];
  __shared__ int kept[64];
  __shared__ int am_last;

  bf16x8 qreg[C::KS];
  load_q<D>(a, b, h, qreg);
  const unsigned short* kb = a.kc + b * a.ksb + h * a.ksh;
  const unsigned short* vb = a.vc + b * a.vsb + h * a.vsh;
  const int v_begin = imin(split * a.rpa, total);
  const int v_end = imin(v_begin + a.rpa, total);
  auto info = [&](int v, int& pos, int& fl) {
    if (v < ntop) {
      pos = pos_of(l, top, v);
      fl = (v < natt ? kAttend : 0) | (v < nsc ? kScore : 0);
    } else if (v < ntop + nsink) {
      pos = v - ntop;
      fl = kAttend;
    } else {
      pos = lo + (v - ntop - nsink);
      fl = kAttend;
    }
  };
  f32x4 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f, l_ex = 0.f;
  stream_rows<D>(v_begin, v_end, info, kb, a.kst, vb, a.vst, qreg, a.c2, lds.stage0, lds.stage1, rowpos, rowflag,
                 ktop > 0 ? rowscore : nullptr, oacc, m_run, l_run, l_ex);
  float* gpart = a.part + gidx * a.nslot * G * (D + kPartExtra);
  store_partial<D>(oacc, m_run, l_run, l_ex, G, wstat, reinterpret_cast<float*>(lds.stage0),
                   gpart + (size_t)split * G * (D + kPartExtra));

  // this split's best candidates (those whose gists it scored; splits start
  // at multiples of `per`, so no candidate straddles two)
  float* gls = a.list_s + gidx * a.nsa * 64;
  int* gli = a.list_i + gidx * a.nsa * 64;
  if (ktop > 0) {
    const int c0 = v_begin / per;
    const int c1 = imax(c0, imin(v_end, nsc) / per);
    float rs;
    int ri;
    rank_candidates(
        c1 - c0,
        [&](int e) {
          float s = 0.f;
          for (int t = 0; t < per; ++t) s += rowscore[(c0 + e) * per + t - v_begin];
          return s * a.score_mul2;
        },
        [&](int e) { return c0 + e; }, lds_s, lds_i, rs, ri);
    if (wave == 0) {
      st_dev(&gls[split * 64 + lane], rs);
      __hip_atomic_store(&gli[split * 64 + lane], ri, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // one level: phase B merges the lists.  Two levels: the last split of this
  // (batch, KV head) makes the group selection and runs the level-1 stage.
  if (!two) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&a.counters[gidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    am_last = prev == a.nsa - 1;
  }
  __syncthreads();
  if (!am_last) return;
  int nkept = 0;
  if (ktop > 0) {
    // merge the splits' lists: wave w takes lists w, w + 4, ... then the tree
    float rs = -__builtin_inff();
    int ri = INT_MAX;
    for (int sp = wave; sp < a.nsa; sp += 4) {
      const float xs = ld_dev(&gls[sp * 64 + lane]);
      const int xi = __hip_atomic_load(&gli[sp * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (sp == wave) {
        rs = xs;
        ri = xi;
      } else {
        wave_merge(rs, ri, xs, xi);
      }
    }
    lds_s[wave * 64 + lane] = rs;
    lds_i[wave * 64 + lane] = ri;
    __syncthreads();
    for (int st = 1; st < 4; st <<= 1) {
      if ((wave & (2 * st - 1)) == 0 && wave + st < 4) {
        wave_merge(rs, ri, lds_s[(wave + st) * 64 + lane], lds_i[(wave + st) * 64 + lane]);
        lds_s[wave * 64 + lane] = rs;
        lds_i[wave * 64 + lane] = ri;
      }
      __syncthreads();
    }
    if (wave == 0) {
      const int nv = place_ascending(lane < ktop ? ri : INT_MAX, ktop, (two ? a.selg + gidx * l.k2 : a.sel + gidx * l.k),
                                     kept);
      if (lane == 0) lds_i[0] = nv;
    }
    __syncthreads();
    nkept = lds_i[0];
  }
  float* extra = gpart + (size_t)a.nsa * G * (D + kPartExtra);

  // two levels: the level-1 gists of the kept groups, scored and (before the
  // window) attended; candidates are every chunk of a kept group (complete,
  // as the group is)
  const int ngr = ncand;
  const int cpg = l.G2;                    // chunks per group
  const int rows_pg = cpg * l.g;           // level-1 gists per group
  const int nl1 = imin(nkept * rows_pg, kMaxL1Rows);
  const int nl1_att = count_below(l, K_GIST, lo);   // level-1 gists before the window
  auto info1 = [&](int v, int& pos, int& fl) {
    const int e = v / rows_pg, t = v - e * rows_pg;
    const int gr = iclamp(kept[e], 0, imax(ngr - 1, 0));
    const int u = gr * rows_pg + t;
    pos = pos_of(l, K_GIST, u);
    fl = kScore | (u < nl1_att ? kAttend : 0);
  };
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  m_run = kNegBig;
  l_run = 0.f;
  l_ex = 0.f;
  stream_rows<D>(0, nl1, info1, kb, a.kst, vb, a.vst, qreg, a.c2, lds.stage0, lds.stage1, rowpos, rowflag, rowscore,
                 oacc, m_run, l_run, l_ex);
  store_partial<D>(oacc, m_run, l_run, l_ex, G, wstat, reinterpret_cast<float*>(lds.stage0), extra);
  float rs;
  int ri;
  rank_candidates(
      nl1 / l.g,
      [&](int e) {
        float s = 0.f;
        for (int t = 0; t < l.g; ++t) s += rowscore[e * l.g + t];
        return s * a.score_mul1;
      },
      [&](int e) {
        const int gi = e / cpg;
        return iclamp(kept[gi], 0, imax(ngr - 1, 0)) * cpg + (e - gi * cpg);
      },
      lds_s, lds_i, rs, ri);
  if (wave == 0) place_ascending(lane < l.k ? ri : INT_MAX, l.k, a.sel + gidx * l.k, nullptr);
  if (tid == 0) __hip_atomic_store(&a.counters[gidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- phase B
template <int D, typename TO>
__global__ __launch_bounds__(kThreads) void k_step_b(StepArgs a) {
  using C = DCfg<D>;
  const Lay& l = a.l;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.Hq / a.Hkv;
  const int i = a.kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);
  const size_t gidx = (size_t)b * a.Hkv + h;

  __shared__ __attribute__((aligned(1024))) StepLds<D> lds;
  __shared__ int rowpos[2][kRows], rowflag[3][kRows];
  __shared__ float wstat[192];
  __shared__ int seg_start[65], seg_base[64];
  __shared__ int chosen[64];
  __shared__ int nseg, am_last;
  const bool two = l.G2 > 0;

  // q first: its loads are in flight while the selection is read
  bf16x8 qreg[C::KS];
  load_q<D>(a, b, h, qreg);
  // unfolded chunks' raws before the window: one contiguous run per chunk,
  // laid out by an exclusive scan over the selection (lanes of wave 0)
  if (wave == 0) {
    const int nch = count_below(l, K_GIST, i) / l.g;   // complete chunks
    int m = -1;
    if (!two) {
      // one level: merge phase A's best-first lists, then the chosen chunks
      // ascending (split 0 also writes them out)
      float rs = -__builtin_inff();
      int ri = INT_MAX;
      const float* gls = a.list_s + gidx * a.nsa * 64;
      const int* gli = a.list_i + gidx * a.nsa * 64;
      for (int sp = 0; sp < a.nsa; ++sp) {
        const float xs = gls[sp * 64 + lane];
        const int xi = gli[sp * 64 + lane];
        if (sp == 0) {
          rs = xs;
          ri = xi;
        } else {
          wave_merge(rs, ri, xs, xi);
        }
      }
      place_ascending(lane < l.k ? ri : INT_MAX, l.k, chosen, nullptr);
      __builtin_amdgcn_wave_barrier();
      if (lane < l.k) {
        m = chosen[lane];
        if (split == 0) a.sel[gidx * l.k + lane] = m;
      }
    } else if (lane < l.k) {
      m = a.sel[gidx * l.k + lane];
    }
    int len = 0, st = 0;
    if (lane < l.k) {
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
    if (lane < 64) {
      seg_start[lane] = incl - len;
      seg_base[lane] = st;
    }
    if (lane == 63) {
      seg_start[64] = incl;
      nseg = 64;
    }
  }
  __syncthreads();
  const int total = seg_start[64];
  auto info = [&](int v, int& pos, int& fl) {
    int lo_s = 0, hi_s = 63;    // last run with start <= v (empty runs are skipped by the search)
    while (lo_s < hi_s) {
      const int mid = (lo_s + hi_s + 1) >> 1;
      if (seg_start[mid] <= v) lo_s = mid;
      else hi_s = mid - 1;
    }
    pos = seg_base[lo_s] + (v - seg_start[lo_s]);
    fl = kAttend;
  };
  const unsigned short* kb = a.kc + b * a.ksb + h * a.ksh;
  const unsigned short* vb = a.vc + b * a.vsb + h * a.vsh;
  const int v_begin = imin(split * a.rpb, total);
  const int v_end = imin(v_begin + a.rpb, total);
  f32x4 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f, l_ex = 0.f;
  stream_rows<D>(v_begin, v_end, info, kb, a.kst, vb, a.vst, qreg, a.c2, lds.stage0, lds.stage1, rowpos, rowflag,
                 nullptr, oacc, m_run, l_run, l_ex);
  constexpr int PS = D + kPartExtra;
  float* gpart = a.part + gidx * a.nslot * G * PS;
  store_partial<D>(oacc, m_run, l_run, l_ex, G, wstat, reinterpret_cast<float*>(lds.stage0),
                   gpart + (size_t)(a.nsa + 1 + split) * G * PS);

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* cnt = a.counters + (size_t)gridDim.z * a.Hkv;   // phase-B counters
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&cnt[gidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    am_last = prev == a.nsb - 1;
  }
  __syncthreads();
  if (!am_last) return;
  // merge every slot (phase A splits, the level-1 slot, phase B splits)
  // (one level has no level-1 partial: its slot, a.nsa, is skipped)
  merge_partials<D, TO>(gpart, a.nslot, G, reinterpret_cast<TO*>(a.o), a.osb, a.osh, a.lse, a.Hq, b, h,
                        two ? -1 : a.nsa);
  if (tid == 0) __hip_atomic_store(&cnt[gidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- planning
struct StepPlan {
  int nsa, rpa, nsb, rpb, nslot;
  size_t off_lists_s, off_lists_i, off_part, bytes;
};

int device_cus() {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return cus;
}

gsa_status plan_step(const Lay& l, int B, int Hq, int Hkv, int d, int kv_len, StepPlan* p) {
  const bool two = l.G2 > 0;
  const int i = kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);
  const int top = two ? K_GIST2 : K_GIST;
  const int per = two ? l.g2 : l.g;
  const int ncand = count_below(l, top, i) / per;
  const int rows_a = imax(count_below(l, top, lo), ncand * per) + imin(l.S, lo) + (i - lo + 1);
  const int groups = imax(1, B * Hkv);
  const int target = 2 * device_cus();   // workgroups per phase: about two per CU
  // phase A: rows per split a multiple of 64 and of `per`, at most kMaxRowsPerSplit
  int ns = iclamp((target + groups - 1) / groups, 1, kMaxSplit);
  ns = imin(ns, imax(1, (rows_a + kRows - 1) / kRows));
  int unit = kRows;
  while (unit % per) unit += kRows;
  int rp = ((rows_a + ns - 1) / ns + unit - 1) / unit * unit;
  if (rp > kMaxRowsPerSplit) {
    rp = kMaxRowsPerSplit / unit * unit;
    if (rp < unit) return fail(GSA_EUNSUPPORTED, "gists per candidate %d too large", per);
  }
  p->rpa = rp;
  p->nsa = imax(1, (rows_a + rp - 1) / rp);
  if (p->nsa > kMaxSplit)
    return fail(GSA_EUNSUPPORTED, "%d rows per (batch, KV head) need more than %d splits", rows_a, kMaxSplit);
  // phase B: at most k * c raw rows
  const int rows_b = l.k * l.c;
  int nb = iclamp((target + groups - 1) / groups, 1, kMaxSplit);
  nb = imin(nb, imax(1, (rows_b + kRows - 1) / kRows));
  p->rpb = imax(kRows, ((rows_b + nb - 1) / nb + kRows - 1) / kRows * kRows);
  p->nsb = imax(1, (rows_b + p->rpb - 1) / p->rpb);
  p->nslot = p->nsa + 1 + p->nsb;
  const size_t cb = ((size_t)2 * groups * sizeof(int) + 255) / 256 * 256;
  const size_t lists = (size_t)groups * p->nsa * 64;
  p->off_lists_s = cb;
  p->off_lists_i = cb + lists * sizeof(float);
  p->off_part = p->off_lists_i + (lists * sizeof(int) + 255) / 256 * 256;
  p->bytes = p->off_part + (size_t)groups * p->nslot * (Hq / Hkv) * (d + kPartExtra) * sizeof(float);
  return GSA_OK;
}

gsa_status check_step(const gsa_layout* layout, const gsa_tensor& q, const gsa_tensor& k_cache,
                      const gsa_tensor& v_cache, const gsa_tensor& o, int B, int Hq, int Hkv, int d, int kv_len,
                      float scale, Lay* l) {
  gsa_status st = make_lay(layout, kv_len, 64, l);
  if (st != GSA_OK) return st;
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k_cache", k_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("v_cache", v_cache, d)) != GSA_OK) return st;
  if ((st = check_tensor("o", o, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k_cache.dtype != GSA_BF16 || v_cache.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "the decode step takes bf16 q and caches");
  if (o.dtype != GSA_F32 && o.dtype != GSA_BF16) return fail(GSA_EINVAL, "o dtype");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (Hq / Hkv > 16) return fail(GSA_EUNSUPPORTED, "more than 16 query heads per KV head");
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (kv_len < 1) return fail(GSA_EINVAL, "kv_len %d < 1", kv_len);
  if (l->k < 1 || l->k > 64) return fail(GSA_EUNSUPPORTED, "top_k %d outside [1, 64]", l->k);
  if (l->G2 > 0 && l->k2 > 64) return fail(GSA_EUNSUPPORTED, "l2_top_k %d > 64", l->k2);
  if (l->G2 > 0 && (long long)l->k2 * l->G2 * l->g > kMaxL1Rows)
    return fail(GSA_EUNSUPPORTED, "l2_top_k * l2_chunks * gists_per_chunk = %lld level-1 rows (at most %d)",
                (long long)l->k2 * l->G2 * l->g, kMaxL1Rows);
  if (l->G2 > 0 && (long long)l->k2 * l->G2 > 64 * 64)
    return fail(GSA_EUNSUPPORTED, "too many level-1 candidates");
  return GSA_OK;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" size_t gsa_decode_step_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                                  int32_t d, int32_t kv_len) {
  Lay l;
  if (make_lay(layout, kv_len, 64, &l) != GSA_OK || kv_len < 1 || B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv) return 0;
  StepPlan p;
  if (plan_step(l, B, Hq, Hkv, d, kv_len, &p) != GSA_OK) return 0;
  return p.bytes;
}

extern "C" gsa_status gsa_decode_step(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache, gsa_tensor v_cache,
                                      gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                      int32_t kv_len, float scale, int32_t* sel, int32_t* sel_groups, void* ws,
                                      size_t ws_bytes, void* stream) {
  Lay l;
  gsa_status st = check_step(layout, q, k_cache, v_cache, o, B, Hq, Hkv, d, kv_len, scale, &l);
  if (st != GSA_OK) return st;
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is NULL with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  StepPlan p;
  if ((st = plan_step(l, B, Hq, Hkv, d, kv_len, &p)) != GSA_OK) return st;
  if (!ws || ws_bytes < p.bytes) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", p.bytes, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GSA_EINVAL, "workspace must be 256-byte aligned");
  char* w = (char*)ws;
  StepArgs a;
  a.l = l;
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
  a.kv_len = kv_len;
  a.c2 = scale * kLog2e;
  const int G = Hq / Hkv;
  a.score_mul1 = scale / (float)(G * l.g);
  a.score_mul2 = l.G2 > 0 ? scale / (float)(G * l.g2) : a.score_mul1;
  a.counters = (int*)w;
  a.list_s = (float*)(w + p.off_lists_s);
  a.list_i = (int*)(w + p.off_lists_i);
  a.part = (float*)(w + p.off_part);
  a.nsa = p.nsa;
  a.rpa = p.rpa;
  a.nsb = p.nsb;
  a.rpb = p.rpb;
  a.nslot = p.nslot;
  a.sel = sel;
  a.selg = sel_groups;
  a.o = o.ptr;
  a.osb = o.stride_b;
  a.osh = o.stride_h;
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  if (d == 128) {
    hipLaunchKernelGGL((k_step_a<128>), dim3(p.nsa, Hkv, B), dim3(kThreads), 0, s, a);
    if (o.dtype == GSA_F32) hipLaunchKernelGGL((k_step_b<128, float>), dim3(p.nsb, Hkv, B), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_step_b<128, unsigned short>), dim3(p.nsb, Hkv, B), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_step_a<64>), dim3(p.nsa, Hkv, B), dim3(kThreads), 0, s, a);
    if (o.dtype == GSA_F32) hipLaunchKernelGGL((k_step_b<64, float>), dim3(p.nsb, Hkv, B), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((k_step_b<64, unsigned short>), dim3(p.nsb, Hkv, B), dim3(kThreads), 0, s, a);
  }
  return launch_status("gsa_decode_step");
}
