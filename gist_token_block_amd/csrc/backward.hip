// Backward pass of the block-sparse prefill on bf16 MFMA (gfx950): dQ, dK, dV
// over the same tile tables as the forward.  The pages train the sparse
// pattern end to end (Forget, Then Recall ... Gist Sparse Attention,
// abstract; the UniGist summary names forward and backward latency among its
// efficiency measures, Experimental setup).  With s = scale q.k, P the
// softmax over the row's visible keys, D_i = dO_i . O_i:
//     dS = P (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// P is recomputed from the forward's log-sum-exp, never stored.
//
// k_bwd_dq: the forward's workgroup shape (4 waves, 128 query rows of one
// query head) walking the row tile's key tiles.  Per tile S^T = K Q^T and
// dP^T = V dO^T (keys on M, queries on N), so dS^T leaves the accumulators
// with a lane's query fixed and becomes the B operand of dQ^T += K^T dS^T, K^T
// read with ds_read_b64_tr_b16 exactly as the forward reads V^T.  K therefore
// sits in LDS in the transposed-read swizzle and V in the row-read one.  The
// kernel also writes D for the second kernel.
//
// k_bwd_dkdv: one workgroup of 8 waves per (batch, KV head, two key tiles);
// each wave owns 16 keys of one tile, holds their K and V rows as MFMA
// operands in registers (v_mfma_f32_16x16x32_bf16, so a wave needs about half
// the registers of a 32-key form and two waves fit a SIMD), and accumulates
// their dK and dV over every row of every stage.
// The stages are the query tiles whose table code for either key tile is
// non-zero, for every query head of the KV group, each cut in two 64-row
// halves; Q, dO, log-sum-exp and D of a stage go through LDS three deep, so
// two stages are loading while one is computed.  S = Q K^T and dP = dO V^T
// are taken with keys on N, so P^T and dS^T leave the accumulators with a
// lane's key fixed and are the A operands of dV += P^T dO and dK += dS^T Q,
// dO and Q read transposed.
//
// Masking: only PARTIAL or short tiles, and only layouts whose visibility in
// a tile is one stream range per query (the fixed layout: sinks, gists and
// the causal window; and block masks, where every key is a sink).
#include "gsa_internal.h"

namespace gsa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kStage = 64;   // query rows per dK/dV stage

template <int D> struct BCfg {
  static constexpr int PPR = D / 8;          // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;       // rows per 1 KB wave load
  static constexpr int NIW = kBN / RPI / 4;  // wave loads per 64-row tile per wave
  static constexpr int KS = D / 16;          // k-steps over d
  static constexpr int MT = D / 32;          // 32-wide d tiles
};
template <int D> __device__ inline int swz_row(int r) { return r & (D / 8 - 1); }
template <int D> __device__ inline int swz_tr(int r) { return (4 * (r & 3)) & (D / 8 - 1); }
// dK/dV stage tiles: read as rows (b128, 8 consecutive rows per phase) and
// transposed (b64, 4 rows x 16 columns per 16-lane group); both patterns hit
// distinct 16-byte slots with these (they depend on row % 8 only).
template <int D> __device__ inline int swz_bw(int r) {
  return D == 128 ? ((4 * (r & 3)) ^ (2 * ((r >> 2) & 1))) : ((2 * (r & 3)) | ((r >> 2) & 1));
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* glb_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

template <typename TO> __device__ inline void put4(TO* p, float a, float b, float c, float d);
template <> __device__ inline void put4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
template <> __device__ inline void put4<unsigned short>(unsigned short* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <typename TO> __device__ inline void put1(TO* p, float a);
template <> __device__ inline void put1<float>(float* p, float a) { *p = a; }
template <> __device__ inline void put1<unsigned short>(unsigned short* p, float a) {
  *p = (unsigned short)(pack_bf16x2(a, 0.f) & 0xffffu);
}

// Transposed-read operand: 8 bf16 of one d (lane % 32 + 32 mt) over the rows
// 16 st + 8 (e / 4) + 4 h2 + e % 4, e = 0..7, of a [rows][D] tile stored in
// the swz_tr swizzle (rows 16 st + r and r share it).
template <int D> __device__ inline bf16x8 tr_operand(const unsigned short* base, int tr_off, int st) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + tr_off + (16 * st) * D));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + tr_off + (16 * st + 8) * D));
  const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wh[0], wh[1]});
}

// Pack accumulator slots 8x .. 8x + 7 to a bf16 operand.
__device__ inline bf16x8 pack8(const f32x16& a, int x) {
  unsigned w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(a[8 * x + 2 * e], a[8 * x + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// Visible stream range [lo, hi) of a `kind` stream for the query at i (the
// layouts served here: one range per query).
__device__ inline void stream_range(const Lay& l, int kind, int i, int& lo, int& hi) {
  hi = count_below(l, kind, i + 1);
  lo = kind == K_RAW ? count_below(l, K_RAW, i - l.W1 + 1) : 0;
}

// ------------------------------------------------------------------ dQ (and D)
template <int D, typename TO, bool OF32>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dq(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh,
    const void* __restrict__ o, int64_t osb, int64_t ost, int64_t osh,
    const unsigned short* __restrict__ dO, int64_t dsb, int64_t dst, int64_t dsh, const float* __restrict__ lse,
    TO* __restrict__ dq, int64_t gsb, int64_t gst, int64_t gsh, float* __restrict__ delta,
    float* __restrict__ lse2_out, int Hq, int Hkv,
    int q_begin, int q_len, int nqt, const int8_t* __restrict__ table, const int* __restrict__ tile_cnt,
    const int* __restrict__ tile_list, const int* __restrict__ sel, const int* __restrict__ selg, float c2,
    float scale, int tmode, int total) {
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(1024))) unsigned short K0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short V0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short K1[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short V1[kBN * D];
  __shared__ int rb[4][kBM];   // per row and stream kind: one past the last visible index
  __shared__ int rlo[kBM];     // per row: first raw inside the window

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int x = blockIdx.x;
  const int per = total >> 3, rem = total & 7, xcd = x & 7;
  const int logical = xcd * per + imin(xcd, rem) + (x >> 3);
  const int G = Hq / Hkv;
  int rest = logical;
  const int gq = rest % G;
  rest /= G;
  const int qd = rest % nqt;
  rest /= nqt;
  const int h = rest % Hkv;
  const int b = rest / Hkv;
  const int qt = nqt - 1 - qd;
  const int hq = h * G + gq;

  const int r = qt * kBM + wave * 32 + n;
  const bool rvalid = r < q_len;
  const int rr = imin(r, q_len - 1);
  const int i = q_begin + rr;

  // Q^T and dO^T operands (B of S^T = K Q^T and dP^T = V dO^T): lane (n, h2)
  // holds d = 8 h2 + 16 ks + 0..7 of its row; D = dO . O from the same slices
  bf16x8 qreg[C::KS], dreg[C::KS];
  float dsum = 0.f;
  {
    const unsigned short* qrow = q + b * qsb + (int64_t)rr * qst + hq * qsh;
    const unsigned short* drow = dO + b * dsb + (int64_t)rr * dst + hq * dsh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = 8 * h2 + 16 * ks;
      u32x4 wq = *reinterpret_cast<const u32x4*>(qrow + d0);
      u32x4 wd = *reinterpret_cast<const u32x4*>(drow + d0);
      float ov[8];
      if constexpr (OF32) {
        const float* orow = reinterpret_cast<const float*>(o) + b * osb + (int64_t)rr * ost + hq * osh + d0;
        const f32x4 a = *reinterpret_cast<const f32x4*>(orow), c = *reinterpret_cast<const f32x4*>(orow + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = a[e];
          ov[4 + e] = c[e];
        }
      } else {
        const unsigned short* orow =
            reinterpret_cast<const unsigned short*>(o) + b * osb + (int64_t)rr * ost + hq * osh + d0;
        const u32x4 w = *reinterpret_cast<const u32x4*>(orow);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[2 * e] = lo_bf16(w[e]);
          ov[2 * e + 1] = hi_bf16(w[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = fmaf(lo_bf16(wd[e]), ov[2 * e], dsum);
        dsum = fmaf(hi_bf16(wd[e]), ov[2 * e + 1], dsum);
      }
      if (!rvalid) {
        wq = u32x4{0u, 0u, 0u, 0u};
        wd = u32x4{0u, 0u, 0u, 0u};
      }
      qreg[ks] = __builtin_bit_cast(bf16x8, wq);
      dreg[ks] = __builtin_bit_cast(bf16x8, wd);
    }
  }
  const float Dlt = dsum + __shfl_xor(dsum, 32);
  const float lse2 = rvalid ? lse[((size_t)b * Hq + hq) * q_len + rr] * kLog2e : 0.f;
  if (rvalid && h2 == 0) {
    delta[((size_t)b * Hq + hq) * q_len + r] = Dlt;
    lse2_out[((size_t)b * Hq + hq) * q_len + r] = lse2;
  }
  if (h2 == 0) {
    const int row = wave * 32 + n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      int lo, hi;
      stream_range(l, s, i, lo, hi);
      rb[s][row] = hi;
      if (s == K_RAW) rlo[row] = lo;
    }
  }   // read only after the first tile's barrier

  const unsigned short* kb = k + b * ksb + h * ksh;
  const unsigned short* vb = v + b * vsb + h * vsh;
  const int t = tmode == 1 ? 0 : (tmode == 2 ? b : b * Hkv + h);
  const size_t trow = (size_t)t * nqt + qt;
  const int cnt = tile_cnt[trow];
  const int* list = tile_list + trow * l.nkt;
  const int8_t* codes = table + trow * l.nkt;

  f32x16 dqacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) dqacc[mt] = f32x16{};

  // Staging (the forward's scheme): K pieces in the transposed-read swizzle,
  // V pieces in the row-read swizzle.
  const int srow = lane / C::PPR, sslot = lane % C::PPR;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int koff[C::NIW], voff[C::NIW];
#pragma unroll
  for (int it = 0; it < C::NIW; ++it) {
    const int row = (wave * C::NIW + it) * C::RPI + srow;
    koff[it] = 8 * (sslot ^ swz_tr<D>(row));
    voff[it] = 8 * (sslot ^ swz_row<D>(row));
  }
  auto fetch = [&](int kt, unsigned short* Kd, unsigned short* Vd, int& slot, int& kind, int& u0, int& width) {
    int u1;
    slot = tile_span(l, kt, kind, u0, u1);
    width = u1 - u0;
    const StreamMap sm = slot_map(l, slot);
#pragma unroll
    for (int it = 0; it < C::NIW; ++it) {
      const int wi = wv * C::NIW + it;
      const int row = wi * C::RPI + srow;
      const int p = map_pos(sm, u0 + imin(row, width - 1));
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(kb + (int64_t)p * kst + koff[it]),
                                       (lds_void_ptr)(Kd + wi * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(vb + (int64_t)p * vst + voff[it]),
                                       (lds_void_ptr)(Vd + wi * 512), 16, 0, 0);
    }
  };

  const int tg = lane >> 4, tj = lane & 15;
  const int tr_row = 4 * (tg >> 1) + (tj >> 2);
  const int tr_piece = 2 * (tg & 1) + ((tj & 3) >> 1);
  const int tr_half = tj & 1;
  int kr_off[C::KS], vr_off[C::KS], tr_off[C::MT];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    kr_off[ks] = n * D + 8 * ((h2 + 2 * ks) ^ swz_tr<D>(n));
    vr_off[ks] = n * D + 8 * ((h2 + 2 * ks) ^ swz_row<D>(n));
    asm volatile("" : "+v"(kr_off[ks]));
    asm volatile("" : "+v"(vr_off[ks]));
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    tr_off[mt] = tr_row * D + 8 * ((4 * mt + tr_piece) ^ swz_tr<D>(tr_row)) + 4 * tr_half;
    asm volatile("" : "+v"(tr_off[mt]));
  }

  // the row's selections (layouts with top-k), for PARTIAL tiles whose
  // visibility depends on them
  const int* selrow = sel ? sel + (((size_t)b * Hkv + h) * q_len + rr) * l.k : nullptr;
  const int* selgrow = selg ? selg + (((size_t)b * Hkv + h) * q_len + rr) * l.k2 : nullptr;
  int nslot = 0, nkind = 0, nu0 = 0, nwidth = 0, ncode = 0, kt_next = 0;
  if (cnt > 0) {
    const int kt0 = list[0];
    fetch(kt0, K0, V0, nslot, nkind, nu0, nwidth);
    ncode = codes[kt0];
    if (cnt > 1) kt_next = list[1];
  }

  auto tile = [&](int idx, const unsigned short* Kb, const unsigned short* Vb, unsigned short* Kn,
                  unsigned short* Vn) {
    const int slot = nslot, kind = nkind, u0 = nu0, width = nwidth, code = ncode;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (idx + 1 < cnt) {
      fetch(kt_next, Kn, Vn, nslot, nkind, nu0, nwidth);
      ncode = codes[kt_next];
      if (idx + 2 < cnt) kt_next = list[idx + 2];
    }
    // S^T = K Q^T and dP^T = V dO^T, keys 0..31 (s0, p0) and 32..63 (s1, p1)
    f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kb + kr_off[ks]);
      const bf16x8 kc = *reinterpret_cast<const bf16x8*>(Kb + kr_off[ks] + 32 * D);
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vb + vr_off[ks]);
      const bf16x8 vc = *reinterpret_cast<const bf16x8*>(Vb + vr_off[ks] + 32 * D);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qreg[ks], s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dreg[ks], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, dreg[ks], p1, 0, 0, 0);
    }
    // visibility: slot j of half hf is key 32 hf + 8 (j / 4) + 4 h2 + j % 4
    unsigned vis = 0xffffffffu;
    if (code != 2 || width < kBN) {
      // Kinds whose visible keys form one stream range per row (sinks,
      // level-2 gists, single-level gists, raws without top-k) take the
      // closed-form bounds; the others follow the row's selection key by key.
      const bool ranged = kind == K_SINK || kind == K_GIST2 || (kind == K_GIST && l.G2 == 0) ||
                          (kind == K_RAW && l.k == 0);
      vis = 0;
      if (code != 0 && ranged) {
        const int row = wave * 32 + n;
        const int khi = iclamp(rb[kind][row] - u0, 0, width);
        const int klo = kind == K_RAW ? iclamp(rlo[row] - u0, 0, width) : 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int key = 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h2 + (j & 3);
          vis |= (unsigned)(key >= klo && key < khi) << j;
        }
      } else if (code != 0) {
        const StreamMap sm = slot_map(l, slot);
#pragma unroll 1
        for (int j = 0; j < 32; ++j) {
          const int key = 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h2 + (j & 3);
          bool vv = key < width;
          if (vv) vv = key_visible(l, i, kind, u0 + key, map_pos(sm, u0 + key), selrow, selgrow);
          vis |= (unsigned)vv << j;
        }
      }
    }
    if (!rvalid) vis = 0;
    // dS^T = P^T (dP^T - D), P^T = exp2(s c2 - lse2); then dQ^T += K^T dS^T
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16& sh = hf ? s1 : s0;
      const f32x16& ph = hf ? p1 : p0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pr = ((vis >> (16 * hf + j)) & 1u) ? __builtin_amdgcn_exp2f(fmaf(sh[j], c2, -lse2)) : 0.f;
        sh[j] = pr * (ph[j] - Dlt);
      }
#pragma unroll
      for (int xx = 0; xx < 2; ++xx) {
        const bf16x8 ds = pack8(sh, xx);
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          dqacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(Kb, tr_off[mt], 2 * hf + xx), ds,
                                                              dqacc[mt], 0, 0, 0);
      }
    }
  };
  for (int idx = 0; idx < cnt; idx += 2) {
    tile(idx, K0, V0, K1, V1);
    if (idx + 1 < cnt) tile(idx + 1, K1, V1, K0, V0);
  }

  // lane holds dQ^T[d][query n], d = 32 mt + 8 (j / 4) + 4 h2 + j % 4
  if (rvalid) {
    TO* grow = dq + b * gsb + (int64_t)r * gst + hq * gsh;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        put4<TO>(grow + 32 * mt + 8 * jj + 4 * h2, dqacc[mt][4 * jj] * scale, dqacc[mt][4 * jj + 1] * scale,
                 dqacc[mt][4 * jj + 2] * scale, dqacc[mt][4 * jj + 3] * scale);
  }
}

// ------------------------------------------------------------------ dK, dV
// s_waitcnt with only the vector-memory count bounded (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima, i.e. not waited on).
template <int N> __device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// v_mfma_f32_16x16x32_bf16 operands: A [m = lane % 16][k = 8 (lane / 16) + e],
// B [k = 8 (lane / 16) + e][n = lane % 16], C [m = 4 (lane / 16) + j][n = lane % 16].
constexpr int kWaves16 = 8;

// Transposed-read B operand of the 16x16x32 products: 8 bf16 of column
// d = lane % 16 + 16 mt over the rows base + (e < 4 ? 4 g + e : 16 + 4 g + e - 4),
// g = lane / 16, of a [rows][D] tile stored in the swz_bw swizzle.
template <int D> __device__ inline bf16x8 tr_pair16(const unsigned short* base, int tr_off, int row0) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + tr_off + row0 * D));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(base + tr_off + (row0 + 16) * D));
  const u32x2 wl = __builtin_bit_cast(u32x2, lo), wh = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{wl[0], wl[1], wh[0], wh[1]});
}

template <int D, typename TO>
__global__ __launch_bounds__(64 * kWaves16, 1) void k_bwd_dkdv(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh,
    const unsigned short* __restrict__ dO, int64_t dsb, int64_t dst, int64_t dsh, const float* __restrict__ lse2,
    const float* __restrict__ delta, TO* __restrict__ dk, int64_t ksb_o, int64_t kst_o, int64_t ksh_o,
    TO* __restrict__ dv, int64_t vsb_o, int64_t vst_o, int64_t vsh_o, int Hq, int Hkv, int q_begin, int q_len,
    int nqt, const int8_t* __restrict__ table, const int* __restrict__ sel, const int* __restrict__ selg, float c2,
    float scale, int tmode, int npair, int total) {
  constexpr int PPR = D / 8, RPI = 64 / PPR;
  constexpr int NIW = kStage / RPI / kWaves16;   // wave loads per tensor per stage
  constexpr int KS = D / 32;                     // k-steps of S and dP
  constexpr int MT = D / 16;                     // 16-wide d tiles of dK and dV
  constexpr int NBUF = 3;
  static_assert(NIW >= 1, "stage rows per wave");
  // Q and dO of a 64-row stage, three deep (two prefetches in flight)
  __shared__ __attribute__((aligned(1024))) unsigned short SB[NBUF * 2 * kStage * D];
  __shared__ __attribute__((aligned(16))) float LB[NBUF][kStage], EB[NBUF][kStage];   // lse log2 e, D

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // XCD-aware order: each XCD (blockIdx % 8) runs a contiguous range of
  // (batch, KV head, key-tile pair), so the workgroups streaming one KV
  // group's Q and dO share an L2, and the pairs of sinks and gists, which see
  // the most query tiles, start first.
  const int xb = blockIdx.x;
  const int per = total >> 3, rem = total & 7, xcd = xb & 7;
  const int logical = xcd * per + imin(xcd, rem) + (xb >> 3);
  const int pair = logical % npair;
  const int h = (logical / npair) % Hkv, b = logical / npair / Hkv;
  const int G = Hq / Hkv;
  // key tiles 2 x and 2 x + 1; wave w takes keys [16 (w & 3), + 16) of tile 2 x + (w >> 2)
  const int kt0 = 2 * pair;
  const int ktw = kt0 + (wave >> 2);
  const bool tile_ok = ktw < l.nkt;
  int kind = 0, u0 = 0, u1 = 0, slot = 0;
  if (tile_ok) slot = tile_span(l, ktw, kind, u0, u1);
  const int width = u1 - u0;
  const StreamMap sm = slot_map(l, slot);
  const int key = 16 * (wave & 3) + col;   // this lane's key (N of S and dP)
  const bool kvalid = tile_ok && key < width;
  const int p_key = kvalid ? map_pos(sm, u0 + key) : 0;

  // K^T and V^T operands (B of S = Q K^T, dP = dO V^T): d = 32 ks + 8 g + 0..7
  bf16x8 kreg[KS], vreg[KS];
  {
    const unsigned short* krow = k + b * ksb + (int64_t)p_key * kst + h * ksh;
    const unsigned short* vrow = v + b * vsb + (int64_t)p_key * vst + h * vsh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 32 * ks + 8 * grp));
      vreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vrow + 32 * ks + 8 * grp));
    }
  }
  f32x4 dkacc[MT], dvacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    dkacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int t = tmode == 1 ? 0 : (tmode == 2 ? b : b * Hkv + h);
  const int8_t* col0 = table + (size_t)t * nqt * l.nkt + kt0;   // codes of tile kt0 (stride nkt)
  const bool has1 = kt0 + 1 < l.nkt;

  const int srow = lane / PPR, sslot = lane % PPR;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int soff[NIW];
#pragma unroll
  for (int it = 0; it < NIW; ++it) soff[it] = 8 * (sslot ^ swz_bw<D>((wave * NIW + it) * RPI + srow));
  // every wave issues exactly NIW * 2 + 1 vector loads per stage (one of them
  // lse or D, or a dummy re-load of lse)
  auto fetch = [&](int r0, int hq, int bi) __attribute__((always_inline)) {
    unsigned short* Qd = SB + bi * 2 * kStage * D;
    unsigned short* Od = Qd + kStage * D;
    const unsigned short* qb = q + b * qsb + hq * qsh;
    const unsigned short* ob = dO + b * dsb + hq * dsh;
#pragma unroll
    for (int it = 0; it < NIW; ++it) {
      const int wi = wv * NIW + it;
      const int rr = imin(r0 + wi * RPI + srow, q_len - 1);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(qb + (int64_t)rr * qst + soff[it]),
                                       (lds_void_ptr)(Qd + wi * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)(ob + (int64_t)rr * dst + soff[it]),
                                       (lds_void_ptr)(Od + wi * 512), 16, 0, 0);
    }
    const int rr = imin(r0 + lane, q_len - 1);
    const size_t ri = ((size_t)b * Hq + hq) * q_len + rr;
    if (wv == 1) __builtin_amdgcn_global_load_lds((glb_void_ptr)(delta + ri), (lds_void_ptr)&EB[bi][0], 4, 0, 0);
    else __builtin_amdgcn_global_load_lds((glb_void_ptr)(lse2 + ri), (lds_void_ptr)&LB[bi][0], 4, 0, 0);
  };

  // A-operand row reads (rows 16 t + col, d = 32 ks + 8 g + 0..7; rows 16 t + r
  // share the swizzle of r) and transposed-read offsets (rows 4 g + col / 4;
  // rows 32 qp + r and 32 qp + 16 + r share it too)
  int ar_off[KS], tr_off[MT];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    ar_off[ks] = col * D + 8 * ((grp + 4 * ks) ^ swz_bw<D>(col));
    asm volatile("" : "+v"(ar_off[ks]));
  }
  {
    const int trow = 4 * grp + (col >> 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      tr_off[mt] = trow * D + 8 * ((2 * mt + ((col & 3) >> 1)) ^ swz_bw<D>(trow)) + 4 * (col & 1);
      asm volatile("" : "+v"(tr_off[mt]));
    }
  }

  // The stage sequence: query tiles where either tile's code is non-zero,
  // descending (scanned 64 at a time by ballot; the codes stay in lanes), then
  // every query head of the group, then both 64-row halves.  Every wave walks
  // the same sequence.  Descending, the workgroups of sink and gist keys,
  // which see every later query, all start at the last query tile and move
  // through Q and dO together, so one copy in L2 serves them all.
  int scan0 = (nqt - 1) / 64 * 64;
  unsigned long long smask = 0ull;
  int c0v = 0, c1v = 0;   // this lane's codes for query tile scan0 + lane
  int s_qt = -1, s_gq = 0, s_half = 0, s_c0 = 0, s_c1 = 0;
  auto find_tile = [&]() __attribute__((always_inline)) -> bool {
    while (smask == 0ull) {
      if (scan0 < 0) return false;
      const int qtl = scan0 + lane;
      c0v = qtl < nqt ? col0[(size_t)qtl * l.nkt] : 0;
      c1v = (qtl < nqt && has1) ? col0[(size_t)qtl * l.nkt + 1] : 0;
      smask = __ballot((c0v | c1v) != 0);
      if (smask == 0ull) scan0 -= 64;
    }
    const int bit = 63 - __builtin_clzll(smask);
    smask &= ~(1ull << bit);
    s_qt = scan0 + bit;
    s_c0 = __shfl(c0v, bit);
    s_c1 = __shfl(c1v, bit);
    if (smask == 0ull) scan0 -= 64;
    return true;
  };
  auto next_stage = [&]() __attribute__((always_inline)) -> bool {
    if (s_qt >= 0) {
      if (++s_half < 2 && s_qt * kBM + kStage * s_half < q_len) return true;
      s_half = 0;
      if (++s_gq < G) return true;
      s_gq = 0;
    }
    return find_tile();
  };

  // Stage e uses buffer e % 3.  A is the stage being computed, B and C the
  // (up to) two in flight behind it: first row and this wave's code.
  int a_r0 = 0, a_cd = 0, b_r0 = 0, b_cd = 0, c_r0 = 0, c_cd = 0;
  int nst = 0;   // stages fetched so far
  bool more = next_stage();
  if (more) {
    a_r0 = s_qt * kBM + kStage * s_half;
    a_cd = (wave >> 2) ? s_c1 : s_c0;
    fetch(a_r0, h * G + s_gq, 0);
    nst = 1;
    more = next_stage();
  }
  if (more) {
    b_r0 = s_qt * kBM + kStage * s_half;
    b_cd = (wave >> 2) ? s_c1 : s_c0;
    fetch(b_r0, h * G + s_gq, 1);
    nst = 2;
    more = next_stage();
  }
  for (int cur = 0; cur < nst; ++cur) {
    const int bi = cur % NBUF;
    // this stage's loads are older than the (at most one) later stage's
    if (cur + 1 < nst) wait_vmcnt<NIW * 2 + 1>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (more) {   // refill the buffer freed by stage cur - 1
      c_r0 = s_qt * kBM + kStage * s_half;
      c_cd = (wave >> 2) ? s_c1 : s_c0;
      fetch(c_r0, h * G + s_gq, nst % NBUF);
      ++nst;
      more = next_stage();
    }
    const int r0 = a_r0, code = a_cd;
    a_r0 = b_r0;
    a_cd = b_cd;
    b_r0 = c_r0;
    b_cd = c_cd;
    // Every wave computes every stage (a wave whose tile has code 0 here masks
    // everything): no divergent path around the accumulators.
    const unsigned short* Qb = SB + bi * 2 * kStage * D;
    const unsigned short* Ob = Qb + kStage * D;
    const bool needmask = code != 2 || width < kBN || r0 + kStage > q_len || !tile_ok;   // wave-uniform
#pragma unroll
    for (int qp = 0; qp < 2; ++qp) {   // 32-row blocks of the stage
      // S = Q K^T and dP = dO V^T for the 16-row blocks 2 qp + tt: lane holds
      // rows 32 qp + 16 tt + 4 g + j, this lane's key
      f32x4 s[2], dp[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int rb = (32 * qp + 16 * tt) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(Qb + rb + ar_off[ks]);
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(Ob + rb + ar_off[ks]);
          s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kreg[ks], s[tt], 0, 0, 0);
          dp[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vreg[ks], dp[tt], 0, 0, 0);
        }
      }
      if (needmask) {
        // visibility bits first (bit 4 tt + j), then a select with static
        // indices: no dynamically indexed register write under divergence
        // Kinds whose visible queries follow closed-form stream ranges use
        // them; the others test the key against the query row's selection.
        const bool ranged = kind == K_SINK || kind == K_GIST2 || (kind == K_GIST && l.G2 == 0) ||
                            (kind == K_RAW && l.k == 0);
        const size_t srow0 = ((size_t)b * Hkv + h) * q_len;
        unsigned m = 0;
        for (int x = 0; x < 8; ++x) {
          const int rr = r0 + 32 * qp + 16 * (x >> 2) + 4 * grp + (x & 3);
          bool ok = code != 0 && kvalid && rr < q_len;
          if (ok && ranged) {
            int lo, hi;
            stream_range(l, kind, q_begin + rr, lo, hi);
            const int u = u0 + key;
            ok = u >= lo && u < hi;
          } else if (ok) {
            ok = key_visible(l, q_begin + rr, kind, u0 + key, p_key, sel + (srow0 + rr) * l.k,
                             selg ? selg + (srow0 + rr) * l.k2 : nullptr);
          }
          m |= (unsigned)ok << x;
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) s[tt][j] = ((m >> (4 * tt + j)) & 1u) ? s[tt][j] : kNegBig;
      }
      // P = exp2(s c2 - lse log2 e), dS = P (dP - D); packed as A operands,
      // element e <-> row 32 qp + (e < 4 ? 4 g + e : 16 + 4 g + e - 4)
      unsigned wp[4], wd[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&LB[bi][32 * qp + 16 * tt + 4 * grp]);
        const f32x4 dl = *reinterpret_cast<const f32x4*>(&EB[bi][32 * qp + 16 * tt + 4 * grp]);
        float pr[4], ds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pr[j] = __builtin_amdgcn_exp2f(fmaf(s[tt][j], c2, -l2[j]));
          ds[j] = pr[j] * (dp[tt][j] - dl[j]);
        }
        wp[2 * tt] = pack_bf16x2(pr[0], pr[1]);
        wp[2 * tt + 1] = pack_bf16x2(pr[2], pr[3]);
        wd[2 * tt] = pack_bf16x2(ds[0], ds[1]);
        wd[2 * tt + 1] = pack_bf16x2(ds[2], ds[3]);
      }
      const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{wp[0], wp[1], wp[2], wp[3]});
      const bf16x8 da = __builtin_bit_cast(bf16x8, u32x4{wd[0], wd[1], wd[2], wd[3]});
      // dV += P^T dO, dK += dS^T Q over the 16-wide d tiles
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        dvacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, tr_pair16<D>(Ob, tr_off[mt], 32 * qp), dvacc[mt], 0, 0,
                                                            0);
        dkacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da, tr_pair16<D>(Qb, tr_off[mt], 32 * qp), dkacc[mt], 0, 0,
                                                            0);
      }
    }
  }

  // lane holds dK[key 16 (w & 3) + 4 g + j][d = 16 mt + col]
  if (tile_ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = 16 * (wave & 3) + 4 * grp + j;
      if (kk < width) {
        const int p = map_pos(sm, u0 + kk);
        TO* krow = dk + b * ksb_o + (int64_t)p * kst_o + h * ksh_o;
        TO* vrow = dv + b * vsb_o + (int64_t)p * vst_o + h * vsh_o;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          put1<TO>(krow + 16 * mt + col, dkacc[mt][j] * scale);
          put1<TO>(vrow + 16 * mt + col, dvacc[mt][j]);
        }
      }
    }
  }
}

}  // namespace
}  // namespace gsa

using namespace gsa;

namespace {

// Shared checks and launches of both entry points.
gsa_status backward_common(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o,
                           gsa_tensor dO, const float* lse, gsa_tensor dq, gsa_tensor dk, gsa_tensor dv, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                           const int32_t* sel, const int32_t* sel_groups, const int8_t* table,
                           const int32_t* tile_cnt, const int32_t* tile_list, int32_t block_m, int32_t block_n,
                           float scale, void* ws, size_t ws_bytes, int tmode_in, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  const bool fixed = l.k == 0 && l.G2 == 0;
  const int tmode = tmode_in == 2 ? 2 : (fixed ? 1 : 0);
  if (!fixed && !sel) return fail(GSA_EINVAL, "sel is required when top_k > 0");
  if (fixed && (sel || sel_groups)) return fail(GSA_EINVAL, "sel given for the fixed layout");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is required with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  if (l.k > 64 || l.k2 > 64) return fail(GSA_EUNSUPPORTED, "top_k and l2_top_k are limited to 64");
  const char* names[8] = {"q", "k", "v", "o", "do", "dq", "dk", "dv"};
  const gsa_tensor* ts[8] = {&q, &k, &v, &o, &dO, &dq, &dk, &dv};
  for (int e = 0; e < 8; ++e)
    if ((st = check_tensor(names[e], *ts[e], d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k.dtype != GSA_BF16 || v.dtype != GSA_BF16 || dO.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "the backward takes bf16 q, k, v and do");
  if (dq.dtype != dk.dtype || dq.dtype != dv.dtype) return fail(GSA_EINVAL, "dq, dk, dv dtypes differ");
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (q_begin < 0 || q_len < 1 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (block_m != kBM || block_n != kBN)
    return fail(GSA_EINVAL, "the backward needs the %dx%d table (got %dx%d)", kBM, kBN, block_m, block_n);
  if (!lse || !table || !tile_cnt || !tile_list) return fail(GSA_EINVAL, "lse or table pointers are NULL");
  const size_t need = 2 * (size_t)B * Hq * q_len * sizeof(float);
  if (!ws || ws_bytes < need) return fail(GSA_EINVAL, "workspace of %zu bytes < %zu", ws_bytes, need);
  const int nqt = (q_len + kBM - 1) / kBM;
  const long long total = (long long)B * Hkv * nqt * (Hq / Hkv);
  const long long kv_total = (long long)B * Hkv * ((l.nkt + 1) / 2);
  if (total > 0x7fffffff || kv_total > 0x7fffffff) return fail(GSA_EUNSUPPORTED, "grid too large");
  hipStream_t s = (hipStream_t)stream;
  const float c2 = scale * kLog2e;
  float* delta = (float*)ws;                              // D = rowsum(dO O)
  float* lse2 = delta + (size_t)B * Hq * q_len;            // lse log2 e
  const bool of32 = o.dtype == GSA_F32;
#define GSA_DQ(D, TO, OF)                                                                                        \
  hipLaunchKernelGGL((k_bwd_dq<D, TO, OF>), dim3((unsigned)total), dim3(kThreads), 0, s, l,                      \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h,                            \
                     (const unsigned short*)k.ptr, k.stride_b, k.stride_t, k.stride_h,                            \
                     (const unsigned short*)v.ptr, v.stride_b, v.stride_t, v.stride_h, (const void*)o.ptr,        \
                     o.stride_b, o.stride_t, o.stride_h, (const unsigned short*)dO.ptr, dO.stride_b, dO.stride_t, \
                     dO.stride_h, lse, (TO*)dq.ptr, dq.stride_b, dq.stride_t, dq.stride_h, delta, lse2, Hq, Hkv,   \
                     q_begin, q_len, nqt, table, tile_cnt, tile_list, sel, sel_groups, c2, scale, tmode, (int)total)
#define GSA_KV(D, TO)                                                                                              \
  hipLaunchKernelGGL((k_bwd_dkdv<D, TO>), dim3((unsigned)kv_total), dim3(64 * kWaves16), 0, s,                 \
                     l, (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h,                           \
                     (const unsigned short*)k.ptr, k.stride_b, k.stride_t, k.stride_h,                              \
                     (const unsigned short*)v.ptr, v.stride_b, v.stride_t, v.stride_h,                              \
                     (const unsigned short*)dO.ptr, dO.stride_b, dO.stride_t, dO.stride_h, lse2, delta, (TO*)dk.ptr, \
                     dk.stride_b, dk.stride_t, dk.stride_h, (TO*)dv.ptr, dv.stride_b, dv.stride_t, dv.stride_h, Hq, \
                     Hkv, q_begin, q_len, nqt, table, sel, sel_groups, c2, scale, tmode, (l.nkt + 1) / 2,        \
                     (int)kv_total)
#define GSA_BW(D, TO)                      \
  do {                                     \
    if (of32) GSA_DQ(D, TO, true);         \
    else GSA_DQ(D, TO, false);             \
    if ((st = launch_status("gsa_attn_prefill_backward (dq)")) != GSA_OK) return st; \
    GSA_KV(D, TO);                         \
  } while (0)
  if (d == 128) {
    if (dq.dtype == GSA_F32) GSA_BW(128, float);
    else GSA_BW(128, unsigned short);
  } else {
    if (dq.dtype == GSA_F32) GSA_BW(64, float);
    else GSA_BW(64, unsigned short);
  }
#undef GSA_BW
#undef GSA_KV
#undef GSA_DQ
  return launch_status("gsa_attn_prefill_backward (dk, dv)");
}

}  // namespace

extern "C" size_t gsa_prefill_backward_workspace_bytes(int32_t B, int32_t Hq, int32_t q_len) {
  if (B < 1 || Hq < 1 || q_len < 0) return 0;
  return 2 * (size_t)B * Hq * q_len * sizeof(float);
}

extern "C" gsa_status gsa_attn_prefill_backward(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                                gsa_tensor o, gsa_tensor dO, const float* lse, gsa_tensor dq,
                                                gsa_tensor dk, gsa_tensor dv, int32_t B, int32_t Hq, int32_t Hkv,
                                                int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                                                const int32_t* sel, const int32_t* sel_groups,
                                                const int8_t* table, const int32_t* tile_cnt,
                                                const int32_t* tile_list, int32_t block_m, int32_t block_n,
                                                float scale, void* ws, size_t ws_bytes, void* stream) {
  return backward_common(layout, q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, d, seq_len, q_begin, q_len, sel,
                         sel_groups, table, tile_cnt, tile_list, block_m, block_n, scale, ws, ws_bytes, 0, stream);
}

extern "C" gsa_status gsa_attn_prefill_blockmask_backward(gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o,
                                                          gsa_tensor dO, const float* lse, gsa_tensor dq,
                                                          gsa_tensor dk, gsa_tensor dv, int32_t B, int32_t Hq,
                                                          int32_t Hkv, int32_t d, int32_t seq_len, int32_t q_begin,
                                                          int32_t q_len, const int8_t* table,
                                                          const int32_t* tile_cnt, const int32_t* tile_list,
                                                          int32_t block_m, int32_t block_n, float scale, void* ws,
                                                          size_t ws_bytes, void* stream) {
  if (seq_len < 1) return fail(GSA_EINVAL, "seq_len %d < 1", seq_len);
  gsa_layout all_sinks{};
  all_sinks.n_sink = seq_len;
  all_sinks.chunk_len = 1;
  all_sinks.gists_per_chunk = 1;
  all_sinks.window = 1;
  return backward_common(&all_sinks, q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, d, seq_len, q_begin, q_len,
                         nullptr, nullptr, table, tile_cnt, tile_list, block_m, block_n, scale, ws, ws_bytes, 2,
                         stream);
}

namespace gsa {
size_t unfold_backward_extra_bytes(const Lay& l, int B, int Hkv, int q_len, int nch);
gsa_status launch_unfold_backward(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k, const gsa_tensor& v,
                                  const gsa_tensor& dO, const gsa_tensor& dq, const gsa_tensor& dk,
                                  const gsa_tensor& dv, int B, int Hq, int Hkv, int q_begin, int q_len,
                                  const int* sel, int nch, float scale, const float* lse2, const float* delta,
                                  char* extra, hipStream_t st, int phase);
}  // namespace gsa

namespace {
size_t fixed_part_bytes(int B, int Hq, int q_len) { return (2 * (size_t)B * Hq * q_len * sizeof(float) + 255) / 256 * 256; }
}  // namespace

extern "C" size_t gsa_prefill_unfolded_backward_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq,
                                                                int32_t Hkv, int32_t seq_len, int32_t q_len) {
  Lay l;
  if (!layout || make_lay(layout, seq_len, 64, &l) != GSA_OK || B < 1 || Hq < 1 || Hkv < 1 || q_len < 0 || l.k < 1)
    return 0;
  const int nch = count_below(l, K_GIST, seq_len) / l.g;
  return fixed_part_bytes(B, Hq, q_len) + unfold_backward_extra_bytes(l, B, Hkv, q_len, imax(nch, 1));
}

extern "C" gsa_status gsa_attn_prefill_unfolded_backward(
    const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o, gsa_tensor dO,
    const float* lse, gsa_tensor dq, gsa_tensor dk, gsa_tensor dv, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
    int32_t seq_len, int32_t q_begin, int32_t q_len, const int32_t* sel, const int8_t* table,
    const int32_t* tile_cnt, const int32_t* tile_list, int32_t block_m, int32_t block_n, float scale, void* ws,
    size_t ws_bytes, void* stream) {
  if (!layout) return fail(GSA_EINVAL, "layout is NULL");
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  if (l.G2 != 0) return fail(GSA_EUNSUPPORTED, "the unfolded backward takes one level");
  if (l.k < 1) return fail(GSA_EINVAL, "top_k must be >= 1 (the fixed layout needs no unfolding)");
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (q_len < 1) return fail(GSA_EINVAL, "q_len %d < 1", q_len);
  const size_t need = gsa_prefill_unfolded_backward_workspace_bytes(layout, B, Hq, Hkv, seq_len, q_len);
  if (need == 0) return fail(GSA_EINVAL, "bad sizes for the unfolded backward");
  if (!ws || ws_bytes < need) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GSA_EINVAL, "workspace must be 256-byte aligned");
  // the fixed part (sinks, earlier gists, window) on the fixed layout's tables
  gsa_layout fixed_layout = *layout;
  fixed_layout.top_k = 0;
  if ((st = backward_common(&fixed_layout, q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, d, seq_len, q_begin, q_len,
                            nullptr, nullptr, table, tile_cnt, tile_list, block_m, block_n, scale, ws, ws_bytes, 0,
                            stream)) != GSA_OK)
    return st;
  // then the unfolded keys' share, from the fixed part's D and base-2 lse
  const float* delta = (const float*)ws;
  const float* lse2 = delta + (size_t)B * Hq * q_len;
  char* extra = (char*)ws + fixed_part_bytes(B, Hq, q_len);
  const int nch = imax(1, count_below(l, K_GIST, seq_len) / l.g);
  hipStream_t s = (hipStream_t)stream;
  if ((st = launch_unfold_backward(l, d, q, k, v, dO, dq, dk, dv, B, Hq, Hkv, q_begin, q_len, sel, nch, scale, lse2,
                                   delta, extra, s, 0)) != GSA_OK)
    return st;
  return launch_unfold_backward(l, d, q, k, v, dO, dq, dk, dv, B, Hq, Hkv, q_begin, q_len, sel, nch, scale, lse2,
                                delta, extra, s, 1);
}
