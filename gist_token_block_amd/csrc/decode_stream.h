// Streaming pieces shared by the fused and compact decode kernels: visible
// rows streamed through LDS in double-buffered 64-row blocks into per-wave
// online-softmax state for all query heads of a KV group (MFMA QK and PV),
// the store of a workgroup's partial, the final log-sum-exp merge of all
// partials of a (batch, KV head), and a 4-wave best-first candidate ranking.
#pragma once

#include <limits.h>

#include "decode_common.h"
#include "select_net.h"

namespace gsa {
namespace dec {

// Row flags of a staged block.
constexpr int kAttend = 1, kScore = 2;

template <int D> struct StepLds {
  unsigned short stage0[2 * kRows * D];
  unsigned short stage1[2 * kRows * D];
};

// Streams virtual rows [v_begin, v_end) through LDS in 64-row blocks (double
// buffered, global_load_lds) and folds them into this wave's online-softmax
// state for all query heads of the group.  rowinfo(v, &pos, &flags) gives the
// cache position of virtual row v and whether it is attended and/or scored;
// rows that are scored get the sum over the query heads of their raw logits
// (q.k) written to rowscore[v - v_begin].
template <int D, typename RowInfo>
__device__ void stream_rows(int v_begin, int v_end, RowInfo rowinfo, const unsigned short* __restrict__ kb,
                            int64_t kst, const unsigned short* __restrict__ vb, int64_t vst,
                            const bf16x8* qreg, float c2, unsigned short* __restrict__ stage0,
                            unsigned short* __restrict__ stage1, int (*rowpos)[kRows], int (*rowflag)[kRows],
                            float* __restrict__ rowscore, f32x4* oacc, float& m_run, float& l_run, float& l_ex) {
  using C = DCfg<D>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nblk = (v_end - v_begin + kRows - 1) / kRows;
  if (nblk <= 0) return;
  const int srow = lane / C::PPR, sslot = lane % C::PPR;
  auto positions = [&](int blk) {
    if (tid < kRows) {
      const int v = v_begin + blk * kRows + tid;
      int pos, fl = 0;
      rowinfo(imin(v, v_end - 1), pos, fl);
      rowpos[blk & 1][tid] = pos;
      rowflag[blk % 3][tid] = v < v_end ? fl : 0;
    }
  };
  auto fetch = [&](int blk, unsigned short* Kd) {
    unsigned short* Vd = Kd + kRows * D;
#pragma unroll
    for (int it = 0; it < C::NIW; ++it) {
      const int wi = wave * C::NIW + it;
      const int row = wi * C::RPI + srow;
      const int p = rowpos[blk & 1][row];
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(kb + (int64_t)p * kst + 8 * (sslot ^ dswz_k<D>(row))),
                                       (lds_void_ptr)(Kd + wi * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(vb + (int64_t)p * vst + 8 * (sslot ^ dswz_v<D>(row))),
                                       (lds_void_ptr)(Vd + wi * 512), 16, 0, 0);
    }
  };
  __syncthreads();   // earlier users of rowpos / staging are done
  positions(0);
  if (nblk > 1) positions(1);
  __syncthreads();
  // the first two blocks are copied at once (both buffers are free), so a
  // workgroup of one or two blocks waits for a single memory latency
  fetch(0, stage0);
  if (nblk > 1) fetch(1, stage1);

  const int tj = lane & 15;
  const int trow = 4 * grp + (tj >> 2);
  int k_off[C::KS], tr_off[C::MT];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int row = 16 * wave + col, pc = grp + 4 * ks;
    k_off[ks] = row * D + 8 * (pc ^ dswz_k<D>(row));
    asm volatile("" : "+v"(k_off[ks]));
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    const int row = 16 * wave + trow, pc = 2 * mt + ((tj & 3) >> 1);
    tr_off[mt] = row * D + 8 * (pc ^ dswz_v<D>(row)) + 4 * (tj & 1);
    asm volatile("" : "+v"(tr_off[mt]));
  }

  auto step = [&](int blk, const unsigned short* Kb, unsigned short* next) {
    // One barrier per block: this wave's copies of blk have landed, every
    // wave is done with blk - 1 (whose staging buffer the next fetch reuses
    // and whose row-flag slot positions(blk + 2) rewrites: flags rotate over
    // three slots, positions over two), and the row table of blk + 1 is set.
    // In block 0 the copies of block 1 (2 NIW loads per wave) may still fly.
    if (blk == 0 && nblk > 1) __builtin_amdgcn_s_waitcnt((2 * C::NIW) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int fl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) fl[e] = rowflag[blk % 3][16 * wave + 4 * grp + e];
    if (blk >= 1 && blk + 1 < nblk) fetch(blk + 1, next);
    if (blk + 2 < nblk) positions(blk + 2);
    const unsigned short* Vb = Kb + kRows * D;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + k_off[ks]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], s, 0, 0, 0);
    }
    // s[e]: key row 16 wave + 4 grp + e of the block, head slot col (zero for
    // slots past the group's heads, whose q rows are zero)
    if (rowscore) {
      bool any = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) any |= (fl[e] & kScore) != 0;
      if (__ballot(any)) {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = s[e];
#pragma unroll
          for (int j = 1; j < 16; j <<= 1) v += xor_lane(v, j);
          t[e] = v;
        }
        if (col == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = blk * kRows + 16 * wave + 4 * grp + e;
            if (fl[e] & kScore) rowscore[r] = t[e];
          }
        }
      }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!(fl[e] & kAttend)) s[e] = -__builtin_inff();
      mx = fmaxf(mx, s[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, -m_new));
    const unsigned w0 = pack_bf16x2(s[0], s[1]), w1 = pack_bf16x2(s[2], s[3]);
    const bf16x2 ones = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
    float ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, 0.f, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, ps, false);
    float pe = (s[0] + s[1]) + (s[2] + s[3]);
    ps += __shfl_xor(ps, 16);
    pe += __shfl_xor(pe, 16);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
      ps = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const auto se = __builtin_amdgcn_permlane32_swap(__float_as_uint(pe), __float_as_uint(pe), false, false);
      pe = __uint_as_float(se[0]) + __uint_as_float(se[1]);
    }
    l_run = l_run * alpha + ps;
    l_ex = l_ex * alpha + pe;
    m_run = m_new;
    const bf16x4 pb = __builtin_bit_cast(bf16x4, u32x2{w0, w1});
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      oacc[mt] *= alpha;
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(Vb + tr_off[mt]));
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, pb), oacc[mt], 0, 0, 0);
    }
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    step(blk, stage0, stage1);
    if (blk + 1 < nblk) step(blk + 1, stage1, stage0);
  }
  __syncthreads();   // staging buffers and row tables are reused by the caller
}

// Merges the 4 waves' online-softmax states into one partial per query head
// and stores it at dst ([G][D + kPartExtra]) with device-scope stores.  The
// staging memory `scratch` (>= 4 * 16 * D floats) is clobbered.
template <int D>
__device__ void store_partial(const f32x4* oacc, float m_run, float l_run, float l_ex, int G, float* wstat,
                              float* scratch, float* __restrict__ dst) {
  using C = DCfg<D>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  constexpr int PS = D + kPartExtra;
  float* cm = wstat;
  float* cl = wstat + 64;
  float* ce = wstat + 128;
  if (grp == 0) {
    cm[wave * 16 + col] = m_run;
    cl[wave * 16 + col] = l_run;
    ce[wave * 16 + col] = l_ex;
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) scratch[(wave * 16 + col) * D + 16 * mt + 4 * grp + e] = oacc[mt][e];
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int hd = x / D, dd = x - hd * D;
    float M = kNegBig;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w * 16 + hd]);
    float L = 0.f, LE = 0.f, O = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(cm[w * 16 + hd] - M);
      L += cl[w * 16 + hd] * f;
      LE += ce[w * 16 + hd] * f;
      O += scratch[(w * 16 + hd) * D + dd] * f;
    }
    st_dev(&dst[hd * PS + dd], O);
    if (dd == 0) {
      st_dev(&dst[hd * PS + D], M);
      st_dev(&dst[hd * PS + D + 1], L);
      st_dev(&dst[hd * PS + D + 2], LE);
    }
  }
  __syncthreads();
}

// Best-first top list of candidates [0, ncand) scored by score(e) with ids
// id(e), merged across the waves that hold candidates; wave 0's lanes hold
// the result (rs, ri).  With at most 64 candidates wave 0 holds them all and
// nothing is merged (no barrier either).
template <typename ScoreFn, typename IdFn>
__device__ void rank_candidates(int ncand, ScoreFn score, IdFn id, float* lds_s, int* lds_i, float& rs, int& ri) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int na = imin(4, (ncand + 63) / 64);   // waves holding candidates
  rs = -__builtin_inff();
  ri = INT_MAX;
  bool empty = true;
  for (int b0 = wave * 64; b0 < ncand; b0 += 4 * 64) {
    const int e = b0 + lane;
    float s = -__builtin_inff();
    int d = INT_MAX;
    if (e < ncand) {
      s = nan_to_neg_inf(score(e));
      d = id(e);
    }
    wave_sort_best_first(s, d);
    if (empty) {
      rs = s;
      ri = d;
      empty = false;
    } else {
      wave_merge(rs, ri, s, d);
    }
  }
  if (na <= 1) return;
  __syncthreads();
  lds_s[wave * 64 + lane] = rs;
  lds_i[wave * 64 + lane] = ri;
  __syncthreads();
  for (int st = 1; st < na; st <<= 1) {
    if ((wave & (2 * st - 1)) == 0 && wave + st < na) {
      wave_merge(rs, ri, lds_s[(wave + st) * 64 + lane], lds_i[(wave + st) * 64 + lane]);
      lds_s[wave * 64 + lane] = rs;
      lds_i[wave * 64 + lane] = ri;
    }
    __syncthreads();
  }
}

// Merges the nslot partials of one (batch, KV head) at gpart ([nslot][G][D +
// kPartExtra], device-scope loads; slot `skip`, if in range, is not one) with
// log-sum-exp weights and writes the output rows of the group's G query heads
// (and their log-sum-exp).
template <int D, typename TO>
__device__ void merge_partials(const float* __restrict__ gpart, int nslot, int G, TO* __restrict__ o, int64_t osb,
                               int64_t osh, float* __restrict__ lse, int Hq, int b, int h, int skip = -1) {
  const int tid = threadIdx.x;
  constexpr int PS = D + kPartExtra;
  for (int x = tid; x < G * D; x += kThreads) {
    const int hd = x / D, dd = x - hd * D;
    float Mr = kNegBig, Lr = 0.f, LEr = 0.f, Or = 0.f;
    for (int sp0 = 0; sp0 < nslot; sp0 += 16) {
      float po[16], pm[16], pl[16], pe[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float* pp = gpart + (imin(sp0 + j, nslot - 1) * G + hd) * PS;
        po[j] = ld_dev(&pp[dd]);
        pm[j] = ld_dev(&pp[D]);
        pl[j] = ld_dev(&pp[D + 1]);
        pe[j] = lse && dd == 0 ? ld_dev(&pp[D + 2]) : 0.f;
      }
      float mb = Mr;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (sp0 + j < nslot && sp0 + j != skip) mb = fmaxf(mb, pm[j]);
      const float al = __builtin_amdgcn_exp2f(Mr - mb);
      Lr *= al;
      LEr *= al;
      Or *= al;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (sp0 + j < nslot && sp0 + j != skip) {
          const float wgt = __builtin_amdgcn_exp2f(pm[j] - mb);
          Lr = fmaf(pl[j], wgt, Lr);
          LEr = fmaf(pe[j], wgt, LEr);
          Or = fmaf(po[j], wgt, Or);
        }
      }
      Mr = mb;
    }
    const float val = Or / Lr;
    TO* orow = o + b * osb + (int64_t)(h * G + hd) * osh;
    if constexpr (sizeof(TO) == 4) {
      orow[dd] = val;
    } else {
      orow[dd] = (TO)(pack_bf16x2(val, 0.f) & 0xffffu);
    }
    if (lse && dd == 0) lse[(size_t)b * Hq + h * G + hd] = (Mr + __log2f(LEr)) * kLn2;
  }
}

}  // namespace dec
}  // namespace gsa
