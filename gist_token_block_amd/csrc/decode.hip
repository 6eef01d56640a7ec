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
// rows are cut into a few long splits (about two workgroups per CU in all);
// one workgroup (4 waves) per (split, KV head, batch) streams its rows in
// 64-row blocks of K and V straight into LDS, double buffered
// (global_load_lds_dwordx4: the next block flies while this one is computed;
// one chunk's raws are
// contiguous in the [B, Hkv, kv_len, d] cache), and each wave takes 16 rows
// of a block for all G query heads of the KV group at once:
//   S^T (16 keys x 16 head slots) = K q^T   v_mfma_f32_16x16x32_bf16
//   O^T (16 d x 16 head slots)   += V^T P^T v_mfma_f32_16x16x16_bf16
// The S accumulator layout (lane = head slot, 4 keys) is exactly the B operand
// layout of the 16x16x16 product, so P never leaves registers; the V^T operand
// comes from the row-major V block through ds_read_b64_tr_b16.  Waves keep
// separate (max, sum, O) partials, merged in LDS into the split's partial; the
// last split of a (batch, KV head) to finish (a counter in the workspace)
// merges all splits with log-sum-exp weights and writes the output.
#include <mutex>

#include "decode_common.h"

namespace gsa {
namespace {
using namespace dec;

// Workspace: int counters [B*Hkv] (zero between calls), then partials
// [B*Hkv][nsplit][G][D + 3] (O, then max in log2 units, then the sum of the
// bf16 P that O is built from, then the sum of the unrounded P, which gives
// the log-sum-exp).
template <int D, typename TO>
__global__ __launch_bounds__(kThreads) void k_decode(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qsh,
    const unsigned short* __restrict__ kc, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ vc, int64_t vsb, int64_t vst, int64_t vsh, int Hq, int Hkv,
    int kv_len, const int* __restrict__ sel, const int* __restrict__ selg, float c2,
    int* __restrict__ counters, float* __restrict__ part, int nsplit, int rows_per_split,
    TO* __restrict__ o, int64_t osb, int64_t osh, float* __restrict__ lse) {
  using C = DCfg<D>;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int G = Hq / Hkv;
  const int i = kv_len - 1;
  const int lo = imax(0, i - l.W1 + 1);
  const size_t gidx = (size_t)b * Hkv + h;

  __shared__ Segs segs;
  __shared__ int rowpos[2][kRows];
  __shared__ int ssel[64], sselg[64];
  __shared__ int am_last;
  __shared__ float wstat[192];
  // Two staging buffers, K then V rows of one block each.  They are separate
  // arrays indexed only statically: the compiler can then tell the prefetch's
  // LDS writes from the reads of the current block and does not make every
  // LDS read wait for the prefetch.
  __shared__ __attribute__((aligned(1024))) unsigned short stage[2 * kRows * D];
  __shared__ __attribute__((aligned(1024))) unsigned short stage1[2 * kRows * D];

  // selections first, all at once (the table build below reads them serially)
  if (tid < l.k) ssel[tid] = sel[gidx * l.k + tid];
  if (selg && tid >= 64 && tid - 64 < l.k2) sselg[tid - 64] = selg[gidx * l.k2 + tid - 64];
  __syncthreads();

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
    if (l.G2 == 0) {
      add(K_GIST, 0, count_below(l, K_GIST, lo));
    } else {
      add(K_GIST2, 0, count_below(l, K_GIST2, lo));
      const int gl = count_below(l, K_GIST, lo), per = l.G2 * l.g;
      const int ngr = count_below(l, K_GIST2, i) / l.g2;   // groups complete before i
      for (int e = 0; e < l.k2; ++e) {
        const int gr = sselg[e];
        if (gr >= 0 && gr < ngr) add(K_GIST, gr * per, iclamp(gl - gr * per, 0, per));
      }
    }
    add(-1, lo, i - lo + 1);
    const int nch = count_below(l, K_GIST, i) / l.g;          // chunks complete before i
    for (int e = 0; e < l.k; ++e) {
      const int m = ssel[e];
      if (m < 0 || m >= nch) continue;   // ids outside the candidates are ignored
      const int st = pos_of(l, K_RAW, m * l.c);
      add(-1, st, iclamp(lo - st, 0, l.c));
    }
    segs.start[n] = tot;
    segs.n = n;
    am_last = 0;
  }
  __syncthreads();
  const int total = segs.start[segs.n];
  const int v_begin = imin(split * rows_per_split, total);
  const int v_end = imin(v_begin + rows_per_split, total);
  const int nblk = (v_end - v_begin + kRows - 1) / kRows;

  const unsigned short* kb = kc + b * ksb + h * ksh;
  const unsigned short* vb = vc + b * vsb + h * vsh;
  const int srow = lane / C::PPR, sslot = lane % C::PPR;
  // Row positions of block `blk` (rows past the end repeat the last one; their
  // logits are masked, so the duplicate never counts), then its K and V rows
  // straight into LDS buffer blk % 2.
  auto positions = [&](int blk) {
    if (tid < kRows) rowpos[blk & 1][tid] = seg_pos(l, segs, imin(v_begin + blk * kRows + tid, v_end - 1));
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
  if (nblk > 0) positions(0);
  if (nblk > 1) positions(1);
  __syncthreads();
  if (nblk > 0) fetch(0, stage);

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
  // transposed-read roles for the V^T operand of the 16x16x16 product: this
  // lane supplies row 4 grp + j/4 (+16 wave), d-chunk 4 (j%4) (+16 mt)
  const int tj = lane & 15;
  const int trow = 4 * grp + (tj >> 2);
  // Per-lane element offsets of the K and V^T operands inside a block.  The
  // empty asm makes each opaque, so every LDS read is one offset from its
  // buffer: the compiler then keeps the buffer's alias scope on it (a long
  // chain of derived addresses loses it, and an unscoped read waits for
  // every copy in flight, the prefetch included).
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
  f32x4 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f, l_ex = 0.f;

  auto step = [&](int blk, const unsigned short* Kb, unsigned short* next) {
    // One barrier per block: this wave's copies of block blk have landed
    // (the wait), so after the barrier all of them have, every wave is done
    // with block blk - 1 (whose buffer the next fetch reuses), and the
    // positions of blk + 1 are set.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 1 < nblk) fetch(blk + 1, next);
    if (blk + 2 < nblk) positions(blk + 2);
    const unsigned short* Vb = Kb + kRows * D;
    const int r0 = 16 * wave;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + k_off[ks]);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], s, 0, 0, 0);
    }
    // s[e]: key row r0 + 4 grp + e of the block, head slot col
    const int vrow0 = v_begin + blk * kRows + r0 + 4 * grp;
    float mx = -__builtin_inff();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (vrow0 + e >= v_end) s[e] = -__builtin_inff();
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
    step(blk, stage, stage1);
    if (blk + 1 < nblk) step(blk + 1, stage1, stage);
  }
  __syncthreads();   // staging memory is reused below

  // ---- merge the 4 waves' partials, write this split's partial
  float* cm = wstat;                                   // [4][16]
  float* cl = wstat + 4 * 16;                          // [4][16]
  float* ce = wstat + 8 * 16;                          // [4][16]
  float* co = reinterpret_cast<float*>(stage);         // [4][16][D]
  static_assert(2 * kRows * D * 2 >= 64 * D * 4, "LDS reuse too small");
  if (grp == 0) {
    cm[wave * 16 + col] = m_run;
    cl[wave * 16 + col] = l_run;
    ce[wave * 16 + col] = l_ex;
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) co[(wave * 16 + col) * D + 16 * mt + 4 * grp + e] = oacc[mt][e];
  __syncthreads();
  constexpr int PS = D + kPartExtra;   // floats per (split, head) partial
  float* mypart = part + (gidx * nsplit + split) * G * PS;
  for (int x = tid; x < G * D; x += kThreads) {
    const int hd = x / D, dd = x - hd * D;
    float M = kNegBig;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w * 16 + hd]);
    float L = 0.f, LE = 0.f, O = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(cm[w * 16 + hd] - M);
      L += cl[w * 16 + hd] * f;
      LE += ce[w * 16 + hd] * f;
      O += co[(w * 16 + hd) * D + dd] * f;
    }
    // device-scope stores: coherent across the XCDs' L2s without a cache-wide
    // write-back (a device-scope fence here costs far more than the kernel)
    st_dev(&mypart[hd * PS + dd], O);
    if (dd == 0) {
      st_dev(&mypart[hd * PS + D], M);
      st_dev(&mypart[hd * PS + D + 1], L);
      st_dev(&mypart[hd * PS + D + 2], LE);
    }
  }

  // ---- the last split of this (batch, KV head) merges all partials: every
  // thread's partial stores have completed before the barrier that precedes
  // the counter update, and the merging workgroup reads them after seeing
  // the count, with device-scope loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(&counters[gidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    am_last = prev == nsplit - 1;
  }
  __syncthreads();
  if (!am_last) return;
  const float* gp = part + gidx * nsplit * G * PS;
  // Each thread merges one (head, d) over all splits, loading every split's
  // partial, max and sum of a batch together (one round trip per 16 splits)
  // and rescaling online between batches.
  for (int x = tid; x < G * D; x += kThreads) {
    const int hd = x / D, dd = x - hd * D;
    float Mr = kNegBig, Lr = 0.f, LEr = 0.f, Or = 0.f;
    for (int sp0 = 0; sp0 < nsplit; sp0 += 16) {
      float po[16], pm[16], pl[16], pe[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {   // all loads of the batch in flight together
        const float* pp = gp + (imin(sp0 + j, nsplit - 1) * G + hd) * PS;
        po[j] = ld_dev(&pp[dd]);
        pm[j] = ld_dev(&pp[D]);
        pl[j] = ld_dev(&pp[D + 1]);
        pe[j] = lse && dd == 0 ? ld_dev(&pp[D + 2]) : 0.f;
      }
      float mb = Mr;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (sp0 + j < nsplit) mb = fmaxf(mb, pm[j]);
      const float a = __builtin_amdgcn_exp2f(Mr - mb);
      Lr *= a;
      LEr *= a;
      Or *= a;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (sp0 + j < nsplit) {
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
  if (tid == 0) __hip_atomic_store(&counters[gidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

size_t counters_bytes(int B, int Hkv) { return ((size_t)B * Hkv * sizeof(int) + 255) / 256 * 256; }

// Splits per (batch, KV head): enough workgroups for about two per CU in total,
// each streaming a long run of 64-row blocks.
int plan_splits(int B, int Hkv, int rows, int* rows_per_split) {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int groups = imax(1, B * Hkv);
  int ns = iclamp((2 * cus + groups - 1) / groups, 1, kMaxSplit);
  ns = imin(ns, imax(1, (rows + kRows - 1) / kRows));
  const int per = (rows + ns - 1) / ns;
  *rows_per_split = (per + kRows - 1) / kRows * kRows;
  return (rows + *rows_per_split - 1) / *rows_per_split;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" size_t gsa_decode_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                             int32_t d, int32_t kv_len) {
  Lay l;
  if (make_lay(layout, kv_len, 64, &l) != GSA_OK || kv_len < 1 || Hkv < 1 || Hq % Hkv) return 0;
  int rps;
  const int ns = plan_splits(B, Hkv, row_bound(l, kv_len), &rps);
  return counters_bytes(B, Hkv) + (size_t)B * Hkv * ns * (Hq / Hkv) * (d + kPartExtra) * sizeof(float);
}

namespace gsa {
namespace {
using namespace dec;

// Argument checks shared by both decode entry points (nothing is launched).
gsa_status check_decode(const gsa_layout* layout, const gsa_tensor& q, const gsa_tensor& k_cache,
                        const gsa_tensor& v_cache, const gsa_tensor& o, int B, int Hq, int Hkv, int d,
                        int kv_len, const int32_t* sel, const int32_t* sel_groups, float scale, Lay* l) {
  gsa_status st = make_lay(layout, kv_len, 64, l);
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
  if (l->k > 64 || l->k2 > 64) return fail(GSA_EUNSUPPORTED, "top_k and l2_top_k are limited to 64");
  if (l->k > 0 && !sel) return fail(GSA_EINVAL, "sel is required when top_k > 0");
  if (l->G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is required with two levels");
  if (l->G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  return GSA_OK;
}

gsa_status launch_decode(const Lay& l, const gsa_tensor& q, const gsa_tensor& k_cache,
                         const gsa_tensor& v_cache, const gsa_tensor& o, float* lse, int B, int Hq, int Hkv,
                         int d, int kv_len, const int32_t* sel, const int32_t* sel_groups, float scale,
                         int* counters, float* part, int ns, int rps, hipStream_t s) {
  const float c2 = scale * kLog2e;
#define GSA_DECODE(D, TO)                                                                             \
  hipLaunchKernelGGL((k_decode<D, TO>), dim3(ns, Hkv, B), dim3(kThreads), 0, s, l,                    \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_h,                            \
                     (const unsigned short*)k_cache.ptr, k_cache.stride_b, k_cache.stride_t,          \
                     k_cache.stride_h, (const unsigned short*)v_cache.ptr, v_cache.stride_b,          \
                     v_cache.stride_t, v_cache.stride_h, Hq, Hkv, kv_len, sel, sel_groups, c2,        \
                     counters, part, ns, rps, (TO*)o.ptr, o.stride_b, o.stride_h, lse)
  if (d == 128) {
    if (o.dtype == GSA_F32) GSA_DECODE(128, float);
    else GSA_DECODE(128, unsigned short);
  } else {
    if (o.dtype == GSA_F32) GSA_DECODE(64, float);
    else GSA_DECODE(64, unsigned short);
  }
#undef GSA_DECODE
  return GSA_OK;
}

// ---- scratch of gsa_attn_decode_noalloc
// One fixed array per GPU (each device holds its own copy until the process
// ends): completion counters in a fixed region at the start, which every call
// leaves at zero, then the split partials of the current call.  Host code
// never uses the array's name as an address: the device address of the
// current GPU's copy comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchCounterBytes = 64u << 10;    // up to 16384 (batch, KV head) pairs
constexpr size_t kScratchBytes = 8u << 20;            // 8 MiB in all
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void k_zero_words(unsigned* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of this GPU's scratch; on the first call on a device its
// counter region is cleared by a fill kernel on `s` (no memset node, so the
// call can sit inside a captured graph).
gsa_status scratch_ptr(hipStream_t s, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GSA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(GSA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    const int n = (int)(kScratchCounterBytes / 4);
    hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, s, (unsigned*)p, n);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(GSA_EHIP, "clearing the scratch counters: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return GSA_OK;
}

}  // namespace
}  // namespace gsa

extern "C" gsa_status gsa_attn_decode(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                                      gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B, int32_t Hq,
                                      int32_t Hkv, int32_t d, int32_t kv_len, const int32_t* sel,
                                      const int32_t* sel_groups, float scale, void* ws, size_t ws_bytes,
                                      void* stream) {
  Lay l;
  gsa_status st = check_decode(layout, q, k_cache, v_cache, o, B, Hq, Hkv, d, kv_len, sel, sel_groups, scale, &l);
  if (st != GSA_OK) return st;
  const size_t need = gsa_decode_workspace_bytes(layout, B, Hq, Hkv, d, kv_len);
  if (!ws || ws_bytes < need) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GSA_EINVAL, "workspace must be 256-byte aligned");
  int rps;
  const int ns = plan_splits(B, Hkv, row_bound(l, kv_len), &rps);
  int* counters = (int*)ws;
  float* part = (float*)((char*)ws + counters_bytes(B, Hkv));
  launch_decode(l, q, k_cache, v_cache, o, lse, B, Hq, Hkv, d, kv_len, sel, sel_groups, scale, counters, part,
                ns, rps, (hipStream_t)stream);
  return launch_status("gsa_attn_decode");
}

extern "C" gsa_status gsa_attn_decode_noalloc(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                                              gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B,
                                              int32_t Hq, int32_t Hkv, int32_t d, int32_t kv_len,
                                              const int32_t* sel, const int32_t* sel_groups, float scale,
                                              void* stream) {
  Lay l;
  gsa_status st = check_decode(layout, q, k_cache, v_cache, o, B, Hq, Hkv, d, kv_len, sel, sel_groups, scale, &l);
  if (st != GSA_OK) return st;
  if ((size_t)B * Hkv * sizeof(int) > kScratchCounterBytes)
    return fail(GSA_EUNSUPPORTED, "batch x KV heads = %lld exceeds the %zu completion counters of the fixed scratch",
                (long long)B * Hkv, kScratchCounterBytes / sizeof(int));
  int rps;
  const int ns = plan_splits(B, Hkv, row_bound(l, kv_len), &rps);
  const size_t part_bytes = (size_t)B * Hkv * ns * (Hq / Hkv) * (d + kPartExtra) * sizeof(float);
  if (part_bytes > kScratchBytes - kScratchCounterBytes)
    return fail(GSA_EUNSUPPORTED, "these sizes need %zu bytes of split partials; the fixed scratch holds %zu",
                part_bytes, kScratchBytes - kScratchCounterBytes);
  hipStream_t s = (hipStream_t)stream;
  char* base = nullptr;
  if ((st = scratch_ptr(s, &base)) != GSA_OK) return st;
  launch_decode(l, q, k_cache, v_cache, o, lse, B, Hq, Hkv, d, kv_len, sel, sel_groups, scale, (int*)base,
                (float*)(base + kScratchCounterBytes), ns, rps, s);
  return launch_status("gsa_attn_decode_noalloc");
}
