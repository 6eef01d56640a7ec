// Block-sparse flash-style prefill on bf16 MFMA (gfx950), and the
// gsa_attn_prefill entry point.
//
// Each query row attends to its visible keys (sinks, earlier gists, causal
// window: UniGist summary, Approach; plus unfolded chunks: Simplified Sparse
// Attention via Gist Tokens, abstract).  The row's visible keys are walked as
// stream-ordered 64-key tiles taken from the block-visibility table, so EMPTY
// tiles cost nothing and only PARTIAL tiles (or short ones) are masked; the
// grouping of gists into one stream stands in for the gist shift the UniGist
// summary describes (Approach).
//
// Workgroup: 4 waves, 128 query rows of one query head; wave w owns rows
// [32w, 32w+32).  Per key tile:
//   * K and V tiles [64 keys][d] go straight from HBM/L2 into LDS with
//     global_load_lds_dwordx4 (no staging registers), double buffered: the
//     next tile streams in while this one is computed.  16-byte pieces are
//     XOR-swizzled per row so both read patterns below are bank-conflict free.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on M, queries on N), so
//     a lane's 32 logits belong to one query: the row max and sum are in-lane
//     plus one exchange between the two lane halves.
//   * Online softmax in base 2 (scale * log2 e folded into one FMA).
//   * O^T += V^T P^T with the same MFMA.  The V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16 (each 16-lane group gathers a
//     4-key x 16-d block and hands every lane one d with 4 keys); P goes from
//     the S accumulators to bf16 operands without leaving registers, the
//     k-index of both operands mapped to the key each lane already holds.
// Work order: blockIdx is remapped so that each XCD (blockIdx % 8) runs a
// contiguous range of (batch, KV head, query tile descending, query head):
// the query heads sharing a KV head and the neighbouring query tiles, which
// read the same gist stream, hit the same L2, and the heaviest tiles start
// first.
#include "gsa_internal.h"

namespace gsa {

gsa_status launch_prefill_rowwave(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k,
                                  const gsa_tensor& v, const gsa_tensor& o, float* lse, int B, int Hq,
                                  int Hkv, int q_begin, int q_len, int bm, int nqt, const int* sel,
                                  const int* selg, const int8_t* table, const int* tile_cnt,
                                  const int* tile_list, float scale, int tmode, hipStream_t st);

namespace {

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;

template <int D> struct Cfg {
  static constexpr int PPR = D / 8;      // 16-byte pieces per key row
  static constexpr int RPI = 64 / PPR;   // key rows per 1 KB wave load
  static constexpr int NIW = kBN / RPI / 4;  // wave loads per tile per wave (K, and again V)
  static constexpr int KS = D / 16;      // k-steps of the QK product
  static constexpr int MT = D / 32;      // 32-row output tiles of O^T
};
// 16-byte piece p of key row r sits at slot p ^ swz(r).
// K: rows of one 8-lane read phase hit 8 different 16-byte slots.  V: the
// 4 rows x 2 pieces of a 16-lane transposed read, and the two 16-lane groups of
// a 32-lane phase, hit disjoint slots.  Both swizzles depend on row % 16
// (K) or row % 4 (V) only, so a lane's read offsets repeat for every tile.
template <int D> __device__ inline int swz_k(int r) { return r & (D / 8 - 1); }
template <int D> __device__ inline int swz_v(int r) { return (4 * (r & 3)) & (D / 8 - 1); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* glb_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

template <typename TO> struct OutStore;
template <> struct OutStore<float> {
  __device__ static void put4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
};
template <> struct OutStore<unsigned short> {
  __device__ static void put4(unsigned short* p, float a, float b, float c, float d) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
  }
};

// LSE: also write the log-sum-exp, normalised by a separate fp32 sum of the
// unrounded probabilities (O keeps the sum of the bf16 P that feeds it).
// INIT: each row starts from a softmax partial over keys outside the table
// (init [B, q_len, Hq, D + 3]: unnormalised O, max in log2 units, sums) --
// the raw tokens its chosen chunks unfold -- instead of from zero.
// Waves per SIMD: 2 at d = 128 (256 VGPRs).  At d = 64 a tile's products are
// half as long against the same softmax work, and more waves hide more of it:
// 4 (128 VGPRs, the LDS of four workgroups; gzip block-mask workload 0.748 ->
// 0.626 ms), or 3 (168 VGPRs) with the LSE, whose extra sum spills at 128.
template <int D, typename TO, bool LSE, bool INIT>
__global__ __launch_bounds__(kThreads, D == 64 ? (LSE ? 3 : 4) : 2) void k_prefill_mfma(
    Lay l, const unsigned short* __restrict__ q, int64_t qsb, int64_t qst, int64_t qsh,
    const unsigned short* __restrict__ k, int64_t ksb, int64_t kst, int64_t ksh,
    const unsigned short* __restrict__ v, int64_t vsb, int64_t vst, int64_t vsh, TO* __restrict__ o,
    int64_t osb, int64_t ost, int64_t osh, float* __restrict__ lse, int Hq, int Hkv, int q_begin,
    int q_len, int nqt, const int* __restrict__ sel, const int* __restrict__ selg,
    const int8_t* __restrict__ table, const int* __restrict__ tile_cnt,
    const int* __restrict__ tile_list, float c2, int tmode, int total, const float* __restrict__ init) {
  using C = Cfg<D>;
  // Double-buffered K and V tiles as four separate arrays, indexed only
  // statically (the tile loop is unrolled by two): the compiler can then tell
  // the prefetch's LDS writes from the reads of the current tile and does not
  // make those reads wait for the prefetch.
  __shared__ __attribute__((aligned(1024))) unsigned short K0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short V0[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short K1[kBN * D];
  __shared__ __attribute__((aligned(1024))) unsigned short V1[kBN * D];
  // Per query row of the tile: stream entries of each kind at or before the
  // row (index = kind), and raws before its window (index 4).  Kept here
  // rather than in registers for the rare masking of partial tiles.
  __shared__ int rbound[5][kBM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;

  // XCD-aware work order
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

  // this lane's query row and its Q^T operands (B operand of S^T = K Q^T)
  const int r = qt * kBM + wave * 32 + n;
  const bool rvalid = r < q_len;
  const int i = q_begin + r;
  bf16x8 qreg[C::KS];
  {
    const unsigned short* qrow = q + b * qsb + (int64_t)imin(r, q_len - 1) * qst + hq * qsh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 8 * h2 + 16 * ks);
      if (!rvalid) w = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (h2 == 0) {
    const int row = wave * 32 + n;
    rbound[K_SINK][row] = count_below(l, K_SINK, i + 1);
    rbound[K_GIST2][row] = l.G2 ? count_below(l, K_GIST2, i + 1) : 0;
    rbound[K_GIST][row] = count_below(l, K_GIST, i + 1);
    rbound[K_RAW][row] = count_below(l, K_RAW, i + 1);
    rbound[4][row] = count_below(l, K_RAW, i - l.W1 + 1);
  }   // read only after the first tile's barrier
  const int* selrow = sel ? sel + (((size_t)b * Hkv + h) * q_len + imin(r, q_len - 1)) * l.k : nullptr;
  const int* selgrow = selg ? selg + (((size_t)b * Hkv + h) * q_len + imin(r, q_len - 1)) * l.k2 : nullptr;

  const unsigned short* kb = k + b * ksb + h * ksh;
  const unsigned short* vb = v + b * vsb + h * vsh;
  const int t = tmode == 1 ? 0 : (tmode == 2 ? b : b * Hkv + h);   // table per (b, KV head) | one | per b
  const size_t trow = (size_t)t * nqt + qt;
  const int cnt = tile_cnt[trow];
  const int* list = tile_list + trow * l.nkt;
  const int8_t* codes = table + trow * l.nkt;

  f32x16 oacc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) oacc[mt] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;
  float l_ex = 0.f;   // LSE only: sum of the unrounded P
  if constexpr (INIT) {
    if (rvalid) {
      // O^T accumulator element j of tile mt holds d = 32 mt + 8 (j / 4) + 4 h2 + j % 4;
      // the two lanes of a query share the max and split the sums (h2 = 0 holds them)
      const float* ip = init + (((size_t)b * q_len + r) * Hq + hq) * (D + 3);
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(ip + 32 * mt + 8 * jj + 4 * h2);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[mt][4 * jj + e] = w[e];
        }
      m_run = ip[D];
      l_run = h2 == 0 ? ip[D + 1] : 0.f;
      l_ex = h2 == 0 ? ip[D + 2] : 0.f;
    }
  }

  // Staging: wave load `wi` (0 .. 4*NIW-1) fills key rows [wi*RPI, wi*RPI+RPI)
  // of a tile; lane -> row wi*RPI + lane / PPR, LDS slot lane % PPR, which
  // holds the row's 16-byte piece slot ^ swz(row).  Rows past a short tile
  // re-read its last row: those keys are masked to -inf, so their P is 0 and
  // the duplicate (finite) values never count.
  const int srow = lane / C::PPR, sslot = lane % C::PPR;
  const int wv = __builtin_amdgcn_readfirstlane(wave);   // wave index as a scalar: uniform addresses stay scalar
  int koff[C::NIW], voff[C::NIW];   // element offset of the piece this lane fetches
#pragma unroll
  for (int it = 0; it < C::NIW; ++it) {
    const int row = (wave * C::NIW + it) * C::RPI + srow;
    koff[it] = 8 * (sslot ^ swz_k<D>(row));
    voff[it] = 8 * (sslot ^ swz_v<D>(row));
  }
  auto fetch = [&](int kt, unsigned short* Kd, unsigned short* Vd, int& slot, int& kind, int& u0,
                   int& width) {
    int u1;
    slot = tile_span(l, kt, kind, u0, u1);
    width = u1 - u0;
    const StreamMap sm = slot_map(l, slot);
    const bool affine = sm.per == 1 && sm.G == (1 << 30);
    if (affine && width == kBN) {
      // Full tile of an affine stream: row r sits at p0 + r * stride1.  Each
      // load is a wave-uniform base (row block it) plus a 32-bit lane offset.
      const int p0 = sm.base + u0 * sm.stride1;
      const unsigned kstep = (unsigned)(sm.stride1 * kst) * 2u, vstep = (unsigned)(sm.stride1 * vst) * 2u;
      // one 64-bit base per tile; the row block and the lane are a 32-bit offset
      const char* kbase = reinterpret_cast<const char*>(kb + (int64_t)p0 * kst);
      const char* vbase = reinterpret_cast<const char*>(vb + (int64_t)p0 * vst);
#pragma unroll
      for (int it = 0; it < C::NIW; ++it) {
        const int wi = wv * C::NIW + it;
        const unsigned rows = (unsigned)(wi * C::RPI);
        const unsigned klane = (rows + (unsigned)srow) * kstep + 2u * (unsigned)koff[it];
        const unsigned vlane = (rows + (unsigned)srow) * vstep + 2u * (unsigned)voff[it];
        __builtin_amdgcn_global_load_lds((glb_void_ptr)(kbase + klane), (lds_void_ptr)(Kd + wi * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((glb_void_ptr)(vbase + vlane), (lds_void_ptr)(Vd + wi * 512), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int it = 0; it < C::NIW; ++it) {
      const int wi = wv * C::NIW + it;
      const int row = wi * C::RPI + srow;
      const int key = imin(row, width - 1);
      const int p = affine ? sm.base + (u0 + key) * sm.stride1 : map_pos(sm, u0 + key);
      const unsigned short* kp = kb + (int64_t)p * kst + koff[it];
      const unsigned short* vp = vb + (int64_t)p * vst + voff[it];
      __builtin_amdgcn_global_load_lds((glb_void_ptr)kp, (lds_void_ptr)(Kd + wi * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_void_ptr)vp, (lds_void_ptr)(Vd + wi * 512), 16, 0, 0);
    }
  };

  // Transposed-read roles for the V^T operand: this lane supplies the address
  // of key row 4(g/2) + j/4 (+16 st, +8 for the second read), d-chunk
  // 16(g%2) + 4(j%4) (+32 mt), where g = lane / 16, j = lane % 16.
  const int tg = lane >> 4, tj = lane & 15;
  const int tr_row = 4 * (tg >> 1) + (tj >> 2);
  const int tr_piece = 2 * (tg & 1) + ((tj & 3) >> 1);
  const int tr_half = tj & 1;
  // Loop-invariant LDS element offsets.  The empty asm makes each opaque, so
  // every LDS read is one offset from its buffer and keeps that buffer's
  // alias scope (reads reached through longer chains of derived addresses
  // lose it and then wait for every copy in flight, the prefetch included).
  int qk_off[C::KS], tr_off[C::MT];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qk_off[ks] = n * D + 8 * ((h2 + 2 * ks) ^ swz_k<D>(n));
    asm volatile("" : "+v"(qk_off[ks]));
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    tr_off[mt] = tr_row * D + 8 * ((4 * mt + tr_piece) ^ swz_v<D>(tr_row)) + 4 * tr_half;
    asm volatile("" : "+v"(tr_off[mt]));
  }

  // Tile ids run one tile ahead of the copies and codes one tile ahead of
  // their use, so neither global load stalls the loop.
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
    // One barrier per tile: this wave's copies of tile idx have landed (the
    // wait), so after the barrier all have, and every wave is done with tile
    // idx - 1, whose buffers the next fetch overwrites.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- S^T = K Q^T: keys 0..31 into s0 first, then keys 32..63 into s1, so
    // the softmax of the first half can start while the second half's MFMAs run.
    // All K operands of the first half are read before its MFMA chain starts,
    // and each second-half read is issued right after a first-half MFMA, so
    // LDS latency overlaps the chain instead of preceding every step.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    bf16x8 ka[C::KS], kc[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(Kb + qk_off[ks]);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {   // rows n and 32 + n share their swizzle
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qreg[ks], s0, 0, 0, 0);
      kc[ks] = *reinterpret_cast<const bf16x8*>(Kb + qk_off[ks] + 32 * D);
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[ks], qreg[ks], s1, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // each first-half MFMA, then
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // a second-half read (it may reuse the MFMA's operand registers)
    }
    // The next tile's copies go out behind this tile's QK products: the
    // scalar tile lookup and the address arithmetic fill the gaps of the
    // dependent MFMA chain instead of following every wave's barrier.
    if (idx + 1 < cnt) {
      fetch(kt_next, Kn, Vn, nslot, nkind, nu0, nwidth);
      ncode = codes[kt_next];
      if (idx + 2 < cnt) kt_next = list[idx + 2];
    }

    // ---- mask (PARTIAL or short tiles only); lane holds keys 8(j/4)+4h2+j%4 (+32)
    if (code != 2 || width < kBN) {
      // Where no selection is involved (sinks, level-2 gists, single-level
      // gists, raws without top-k) a row's visible keys in a tile form one
      // range of stream indices: those at or before the query, and for raws
      // also inside the window.  Both ends come in closed form.
      const bool ranged = kind == K_SINK || kind == K_GIST2 || (kind == K_GIST && l.G2 == 0) ||
                          (kind == K_RAW && l.k == 0);
      int klo = 0, khi = width;
      if (code != 2 && ranged) {
        const int row = wave * 32 + n;
        khi = iclamp(rbound[kind][row] - u0, 0, width);
        if (kind == K_RAW) klo = iclamp(rbound[4][row] - u0, 0, width);
      }
      unsigned vis = 0;   // bit j: key of s0[j]; bit 16 + j: key of s1[j]
      if (code == 2 || ranged) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int key = 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h2 + (j & 3);
          vis |= (unsigned)(key >= klo && key < khi) << j;
        }
      } else {
        // selection-dependent visibility, key by key (a compact loop)
#pragma unroll 1
        for (int j = 0; j < 32; ++j) {
          const int key = 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h2 + (j & 3);
          bool vv = key < width;
          if (vv) vv = key_visible(l, i, kind, u0 + key, map_pos(slot_map(l, slot), u0 + key), selrow, selgrow);
          vis |= (unsigned)vv << j;
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (!((vis >> j) & 1u)) s0[j] = -__builtin_inff();
        if (!((vis >> (16 + j)) & 1u)) s1[j] = -__builtin_inff();
      }
    }

    // ---- per half: online softmax (base 2), then O^T += V^T P^T for its 32 keys
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16& sh = half ? s1 : s0;
      // V^T operands of this half first: their LDS latency hides behind the
      // softmax below.
      s16x4 vlo[C::MT][2], vhi[C::MT][2];
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int st = 2 * half + x;   // rows 16 st + tr_row (+8) share the swizzle of tr_row
          vlo[mt][x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(Vb + tr_off[mt] + (16 * st) * D));
          vhi[mt][x] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(Vb + tr_off[mt] + (16 * st + 8) * D));
        }
      }
      // P = exp2(s c2 - m_run), packed to bf16 as the PV operand; the row sum
      // adds the bf16-rounded P actually fed to the PV product, so numerator
      // and normaliser use the same weights.  (Packed words stay in scalars:
      // bit-casting elements of a u32x4 here made the compiler feed the first
      // element to every dot2.)
      bf16x8 pk[2];
      float psum, pex;
      auto expo = [&]() {
        psum = 0.f;
        pex = 0.f;
        const bf16x2 ones = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          unsigned w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 8 * x + 2 * e;
            const float pa = __builtin_amdgcn_exp2f(fmaf(sh[j], c2, -m_run));
            const float pb = __builtin_amdgcn_exp2f(fmaf(sh[j + 1], c2, -m_run));
            w[e] = pack_bf16x2(pa, pb);
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, psum, false);
            if constexpr (LSE) pex += pa + pb;
          }
          pk[x] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
      };
      // Lazy rescale without a max on the common path: P is taken against the
      // running reference m_run straight away.  While no lane's sum exceeds
      // 256, every P is at most 256, which bf16 and the fp32 sums hold without
      // loss.  Otherwise (the first tile, or scores well above the reference)
      // the row max is taken, m_run moves up to it, O and the sum are
      // rescaled, and P is recomputed.
      expo();
      if (__ballot(!(psum <= 256.f))) {
        float mx = sh[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sh[j]);
        {  // max with the other half-wave (same queries, the other 16 keys)
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float m_up = fmaxf(m_run, mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_up);
        l_run *= alpha;
        if constexpr (LSE) l_ex *= alpha;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) oacc[mt] *= alpha;
        m_run = m_up;
        expo();
      }
      l_run += psum;
      if constexpr (LSE) l_ex += pex;

      // O^T += V^T P^T; operand element e <-> key 16 st + 8(e/4) + 4 h2 + e%4
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const u32x2 wl = __builtin_bit_cast(u32x2, vlo[mt][x]), wh = __builtin_bit_cast(u32x2, vhi[mt][x]);
          const u32x4 w = u32x4{wl[0], wl[1], wh[0], wh[1]};
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pk[x],
                                                             oacc[mt], 0, 0, 0);
        }
      }
    }
  };
  for (int idx = 0; idx < cnt; idx += 2) {
    tile(idx, K0, V0, K1, V1);
    if (idx + 1 < cnt) tile(idx + 1, K1, V1, K0, V0);
  }

  // ---- normalise and store: lane holds O^T[d][query n], d = 32mt + 8(j/4) + 4h2 + j%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (rvalid) {
    const float inv = 1.f / l_tot;
    TO* orow = o + b * osb + (int64_t)r * ost + hq * osh;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * mt + 8 * jj + 4 * h2;
        OutStore<TO>::put4(orow + d0, oacc[mt][4 * jj] * inv, oacc[mt][4 * jj + 1] * inv,
                           oacc[mt][4 * jj + 2] * inv, oacc[mt][4 * jj + 3] * inv);
      }
    }
    if constexpr (LSE) {
      const float l_ex_tot = l_ex + __shfl_xor(l_ex, 32);
      if (h2 == 0) lse[((size_t)b * Hq + hq) * q_len + r] = (m_run + __log2f(l_ex_tot)) * kLn2;
    }
  }
}

}  // namespace
}  // namespace gsa

using namespace gsa;

namespace {
// Table modes: 0 one table per (batch, KV head) (selections), 1 one table for
// all (the fixed layout), 2 one table per batch entry (block masks).
gsa_status prefill_common(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o,
                          float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                          int32_t q_begin, int32_t q_len, const int32_t* sel, const int32_t* sel_groups,
                          const int8_t* table, const int32_t* tile_cnt, const int32_t* tile_list,
                          int32_t block_m, int32_t block_n, float scale, int tmode_in, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k", k, d)) != GSA_OK) return st;
  if ((st = check_tensor("v", v, d)) != GSA_OK) return st;
  if ((st = check_tensor("o", o, d)) != GSA_OK) return st;
  if (q.dtype != k.dtype || q.dtype != v.dtype) return fail(GSA_EINVAL, "q, k, v dtypes differ");
  if (o.dtype != GSA_F32 && o.dtype != q.dtype) return fail(GSA_EINVAL, "o dtype must be F32 or the input dtype");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (d < 8 || d % 8) return fail(GSA_EUNSUPPORTED, "head dim %d (multiple of 8 required)", d);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (block_m < 1) return fail(GSA_EINVAL, "block_m %d < 1", block_m);
  const bool fixed = l.k == 0 && l.G2 == 0;
  const int tmode = tmode_in == 2 ? 2 : (fixed ? 1 : 0);
  if (!fixed && !sel) return fail(GSA_EINVAL, "sel is required when top_k > 0");
  if (fixed && sel) return fail(GSA_EINVAL, "sel given for the fixed layout");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is required with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  if (l.k > 64 || l.k2 > 64) return fail(GSA_EUNSUPPORTED, "top_k and l2_top_k are limited to 64");
  if (!table || !tile_cnt || !tile_list) return fail(GSA_EINVAL, "table pointers are NULL");
  const int nqt = (q_len + block_m - 1) / block_m;
  hipStream_t s = (hipStream_t)stream;
  const bool mfma = q.dtype == GSA_BF16 && (d == 64 || d == 128);
  if (mfma) {
    if (block_m != kBM || block_n != kBN)
      return fail(GSA_EINVAL, "bf16 d=%d prefill needs a %dx%d table (got %dx%d)", d, kBM, kBN, block_m, block_n);
    const long long total = (long long)B * Hkv * nqt * (Hq / Hkv);
    if (total > 0x7fffffff) return fail(GSA_EUNSUPPORTED, "grid too large");
    const float c2 = scale * kLog2e;
#define GSA_MFMA1(D, TO, LSE)                                                                        \
  hipLaunchKernelGGL((k_prefill_mfma<D, TO, LSE, false>), dim3((unsigned)total), dim3(kThreads), 0, s, l, \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h,                \
                     (const unsigned short*)k.ptr, k.stride_b, k.stride_t, k.stride_h,                \
                     (const unsigned short*)v.ptr, v.stride_b, v.stride_t, v.stride_h, (TO*)o.ptr,    \
                     o.stride_b, o.stride_t, o.stride_h, lse, Hq, Hkv, q_begin, q_len, nqt, sel,      \
                     sel_groups, table, tile_cnt, tile_list, c2, tmode, (int)total, nullptr)
#define GSA_MFMA(D, TO)             \
  if (lse) GSA_MFMA1(D, TO, true);  \
  else GSA_MFMA1(D, TO, false)
    if (d == 128) {
      if (o.dtype == GSA_F32) GSA_MFMA(128, float);
      else GSA_MFMA(128, unsigned short);
    } else {
      if (o.dtype == GSA_F32) GSA_MFMA(64, float);
      else GSA_MFMA(64, unsigned short);
    }
#undef GSA_MFMA
#undef GSA_MFMA1
    return launch_status("gsa_attn_prefill (mfma)");
  }
  if (block_n > 256) return fail(GSA_EUNSUPPORTED, "block_n %d > 256 on the row-wave path", block_n);
  return launch_prefill_rowwave(l, d, q, k, v, o, lse, B, Hq, Hkv, q_begin, q_len, block_m, nqt, sel,
                                sel_groups, table, tile_cnt, tile_list, scale, tmode, s);
}
}  // namespace

extern "C" gsa_status gsa_attn_prefill(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                       gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                                       const int32_t* sel, const int32_t* sel_groups,
                                       const int8_t* table, const int32_t* tile_cnt,
                                       const int32_t* tile_list, int32_t block_m, int32_t block_n,
                                       float scale, void* stream) {
  return prefill_common(layout, q, k, v, o, lse, B, Hq, Hkv, d, seq_len, q_begin, q_len, sel, sel_groups, table,
                        tile_cnt, tile_list, block_m, block_n, scale, 0, stream);
}

extern "C" gsa_status gsa_attn_prefill_blockmask(gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o, float* lse,
                                                 int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                                                 int32_t q_begin, int32_t q_len, const int8_t* table,
                                                 const int32_t* tile_cnt, const int32_t* tile_list,
                                                 int32_t block_m, int32_t block_n, float scale, void* stream) {
  // Every position a sink: the key stream is the physical order, and a sink
  // is visible exactly to the queries at or after it, so PARTIAL tiles get
  // the causal mask and the table carries the block mask.
  if (seq_len < 1) return fail(GSA_EINVAL, "seq_len %d < 1", seq_len);
  gsa_layout all_sinks{};
  all_sinks.n_sink = seq_len;
  all_sinks.chunk_len = 1;
  all_sinks.gists_per_chunk = 1;
  all_sinks.window = 1;
  return prefill_common(&all_sinks, q, k, v, o, lse, B, Hq, Hkv, d, seq_len, q_begin, q_len, nullptr, nullptr,
                        table, tile_cnt, tile_list, block_m, block_n, scale, 2, stream);
}

namespace gsa {
gsa_status launch_unfold(const Lay& l, int d, const gsa_tensor& q, const gsa_tensor& k, const gsa_tensor& v, int B,
                         int Hq, int Hkv, int q_begin, int q_len, const int* sel, float scale, float* part,
                         hipStream_t st);
}

extern "C" size_t gsa_prefill_unfolded_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int32_t q_len) {
  if (B < 1 || Hq < 1 || d < 1 || q_len < 0) return 0;
  return (size_t)B * q_len * Hq * (d + 3) * sizeof(float);
}

extern "C" gsa_status gsa_attn_prefill_unfolded(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                                gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv,
                                                int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                                                const int32_t* sel, const int8_t* table, const int32_t* tile_cnt,
                                                const int32_t* tile_list, int32_t block_m, int32_t block_n,
                                                float scale, void* ws, size_t ws_bytes, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  if (l.G2 != 0) return fail(GSA_EUNSUPPORTED, "unfolded prefill takes one level");
  if (l.k < 1) return fail(GSA_EINVAL, "top_k must be >= 1 (the fixed layout needs no unfolding)");
  gsa_layout fixed_layout = *layout;
  fixed_layout.top_k = 0;
  Lay lf;
  if ((st = make_lay(&fixed_layout, seq_len, block_n, &lf)) != GSA_OK) return st;
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if ((st = check_tensor("q", q, d)) != GSA_OK) return st;
  if ((st = check_tensor("k", k, d)) != GSA_OK) return st;
  if ((st = check_tensor("v", v, d)) != GSA_OK) return st;
  if ((st = check_tensor("o", o, d)) != GSA_OK) return st;
  if (q.dtype != GSA_BF16 || k.dtype != GSA_BF16 || v.dtype != GSA_BF16)
    return fail(GSA_EUNSUPPORTED, "unfolded prefill takes bf16 q, k, v");
  if (o.dtype != GSA_F32 && o.dtype != GSA_BF16) return fail(GSA_EINVAL, "o dtype must be F32 or BF16");
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(GSA_EINVAL, "bad head counts B=%d Hq=%d Hkv=%d", B, Hq, Hkv);
  if (d != 64 && d != 128) return fail(GSA_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d);
  if (!(scale > 0.f)) return fail(GSA_EINVAL, "scale must be > 0");
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (block_m != kBM || block_n != kBN)
    return fail(GSA_EINVAL, "the unfolded prefill needs the %dx%d table of the fixed layout (got %dx%d)", kBM, kBN,
                block_m, block_n);
  if (!sel) return fail(GSA_EINVAL, "sel is NULL");
  if (!table || !tile_cnt || !tile_list) return fail(GSA_EINVAL, "table pointers are NULL");
  const size_t need = gsa_prefill_unfolded_workspace_bytes(B, Hq, d, q_len);
  if (!ws || ws_bytes < need) return fail(GSA_EINVAL, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(GSA_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float* part = (float*)ws;
  if ((st = launch_unfold(l, d, q, k, v, B, Hq, Hkv, q_begin, q_len, sel, scale, part, s)) != GSA_OK) return st;
  const int nqt = (q_len + kBM - 1) / kBM;
  const long long total = (long long)B * Hkv * nqt * (Hq / Hkv);
  if (total > 0x7fffffff) return fail(GSA_EUNSUPPORTED, "grid too large");
  const float c2 = scale * kLog2e;
#define GSA_MFMA_I(D, TO, LSE)                                                                        \
  hipLaunchKernelGGL((k_prefill_mfma<D, TO, LSE, true>), dim3((unsigned)total), dim3(kThreads), 0, s, lf, \
                     (const unsigned short*)q.ptr, q.stride_b, q.stride_t, q.stride_h,                \
                     (const unsigned short*)k.ptr, k.stride_b, k.stride_t, k.stride_h,                \
                     (const unsigned short*)v.ptr, v.stride_b, v.stride_t, v.stride_h, (TO*)o.ptr,    \
                     o.stride_b, o.stride_t, o.stride_h, lse, Hq, Hkv, q_begin, q_len, nqt, nullptr,  \
                     nullptr, table, tile_cnt, tile_list, c2, 1, (int)total, part)
#define GSA_MFMA_I2(D, TO)              \
  if (lse) GSA_MFMA_I(D, TO, true);     \
  else GSA_MFMA_I(D, TO, false)
  if (d == 128) {
    if (o.dtype == GSA_F32) GSA_MFMA_I2(128, float);
    else GSA_MFMA_I2(128, unsigned short);
  } else {
    if (o.dtype == GSA_F32) GSA_MFMA_I2(64, float);
    else GSA_MFMA_I2(64, unsigned short);
  }
#undef GSA_MFMA_I2
#undef GSA_MFMA_I
  return launch_status("gsa_attn_prefill_unfolded");
}
