// Block-visibility table over stream-ordered key tiles (gsa_build_layout).
//
// Visibility: sinks, every earlier gist, a causal window including the query
// (UniGist summary, Approach), plus the raw tokens of the query's unfolded
// chunks (Simplified Sparse Attention via Gist Tokens, abstract) and, with two
// levels, every level-2 gist and the level-1 gists of the kept groups (Forget,
// Then Recall ... Gist Sparse Attention, abstract).
//
// One workgroup per (table, query tile).  Each query row is reduced to a few
// stream-index intervals (what it sees of each stream); a thread then counts
// the visible cells of one key tile by interval overlap, row by row, and the
// tile is coded 0 / 1 / 2.  A block-wide ballot scan compacts the non-empty
// tile ids into the row's list.
#include "gsa_internal.h"

namespace gsa {

namespace {

constexpr int kThreads = 256;

// Per-row intervals, stream-index space.
struct RowInfo {
  int sink_hi;   // sinks visible: [0, sink_hi)
  int g2_hi;     // level-2 gists visible: [0, g2_hi)
  int g_hi;      // gists at positions <= i: [0, g_hi)
  int g_wlo;     // gists inside the window: [g_wlo, g_hi)
  int r_hi;      // raws at positions <= i
  int r_wlo;     // raws inside the window: [r_wlo, r_hi)
};

__global__ __launch_bounds__(kThreads) void k_build_table(Lay l, int q_begin, int q_len, int bm,
                                                          int nqt, const int* __restrict__ sel,
                                                          const int* __restrict__ selg,
                                                          int8_t* __restrict__ table,
                                                          int* __restrict__ tile_cnt,
                                                          int* __restrict__ tile_list) {
  extern __shared__ int smem[];
  const int qt = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  const int r0 = qt * bm;
  const int nrows = imin(bm, q_len - r0);
  RowInfo* rows = reinterpret_cast<RowInfo*>(smem);
  int* ssel = reinterpret_cast<int*>(rows + bm);      // [nrows][k]
  int* sselg = ssel + bm * l.k;                       // [nrows][k2]
  __shared__ int wsum[kThreads / 64];

  for (int r = tid; r < nrows; r += kThreads) {
    const int i = q_begin + r0 + r;
    const int lo = imax(0, i - l.W1 + 1);
    RowInfo ri;
    ri.sink_hi = count_below(l, K_SINK, i + 1);
    ri.g2_hi = l.G2 ? count_below(l, K_GIST2, i + 1) : 0;
    ri.g_hi = count_below(l, K_GIST, i + 1);
    ri.g_wlo = count_below(l, K_GIST, lo);
    ri.r_hi = count_below(l, K_RAW, i + 1);
    ri.r_wlo = count_below(l, K_RAW, lo);
    rows[r] = ri;
  }
  if (sel) {
    const int* src = sel + ((size_t)t * q_len + r0) * l.k;
    for (int e = tid; e < nrows * l.k; e += kThreads) ssel[e] = src[e];
  }
  if (selg) {
    const int* src = selg + ((size_t)t * q_len + r0) * l.k2;
    for (int e = tid; e < nrows * l.k2; e += kThreads) sselg[e] = src[e];
  }
  __syncthreads();

  const size_t row_base = ((size_t)t * nqt + qt) * l.nkt;
  const int lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int base = 0; base < l.nkt; base += kThreads) {
    const int kt = base + tid;
    int code = 0;
    if (kt < l.nkt) {
      int kind, u0, u1;
      tile_span(l, kt, kind, u0, u1);
      // Without a selection each row sees one interval [lo_r, hi_r) of the
      // stream; both ends are non-decreasing in r (by at most one per row), so
      // the first and last rows decide FULL, and a tile is EMPTY unless some
      // row reaching it has a non-empty interval.
      const bool is_raw = kind == K_RAW;
      const bool ranged = kind == K_SINK || kind == K_GIST2 || (kind == K_GIST && l.G2 == 0) ||
                          (is_raw && l.k == 0);
      if (ranged) {
        auto hi_of = [&](const RowInfo& ri) {
          return kind == K_SINK ? ri.sink_hi : kind == K_GIST2 ? ri.g2_hi : kind == K_GIST ? ri.g_hi : ri.r_hi;
        };
        const RowInfo first = rows[0], last = rows[nrows - 1];
        const int lo_first = is_raw ? first.r_wlo : 0, lo_last = is_raw ? last.r_wlo : 0;
        if (lo_last <= u0 && hi_of(first) >= u1) {
          code = 2;
        } else if (hi_of(last) <= u0 || lo_first >= u1) {
          code = 0;
        } else if (!is_raw) {
          code = 1;
        } else {
          // rows [ra, rb) reach the tile: r_hi > u0 from ra on, r_wlo < u1 before rb
          int a = 0, b = nrows;
          while (a < b) {
            const int m = (a + b) >> 1;
            if (rows[m].r_hi > u0) b = m; else a = m + 1;
          }
          const int ra = a;
          a = ra; b = nrows;
          while (a < b) {
            const int m = (a + b) >> 1;
            if (rows[m].r_wlo >= u1) b = m; else a = m + 1;
          }
          code = 0;
          for (int r = ra; r < a; ++r)
            if (rows[r].r_wlo < rows[r].r_hi) { code = 1; break; }
        }
        table[row_base + kt] = (int8_t)code;
      } else {
      int cnt = 0;
      for (int r = 0; r < nrows; ++r) {
        const RowInfo ri = rows[r];
        if (kind == K_SINK) {
          cnt += overlap(u0, u1, 0, ri.sink_hi);
        } else if (kind == K_GIST2) {
          cnt += overlap(u0, u1, 0, ri.g2_hi);
        } else if (kind == K_GIST && l.G2 == 0) {
          cnt += overlap(u0, u1, 0, ri.g_hi);
        } else if (kind == K_GIST) {
          // window part plus the gists of each kept group (not yet counted)
          const int a0 = ri.g_wlo, a1 = ri.g_hi;
          cnt += overlap(u0, u1, a0, a1);
          const int per = l.G2 * l.g;
          for (int e = 0; e < l.k2; ++e) {
            const int gr = sselg[r * l.k2 + e];
            if (gr < 0 || gr >= l.L) continue;
            const int b0 = gr * per, b1 = imin((gr + 1) * per, ri.g_hi);
            cnt += overlap(u0, u1, b0, b1) - overlap(imax(u0, a0), imin(u1, a1), b0, b1);
          }
        } else {
          const int a0 = ri.r_wlo, a1 = ri.r_hi;
          cnt += overlap(u0, u1, a0, a1);
          for (int e = 0; e < l.k; ++e) {
            const int m = sel ? ssel[r * l.k + e] : -1;
            if (m < 0 || m >= l.L) continue;
            const int b0 = m * l.c, b1 = imin((m + 1) * l.c, ri.r_hi);
            cnt += overlap(u0, u1, b0, b1) - overlap(imax(u0, a0), imin(u1, a1), b0, b1);
          }
        }
      }
      const int area = nrows * (u1 - u0);
      code = cnt == 0 ? 0 : (cnt == area ? 2 : 1);
      table[row_base + kt] = (int8_t)code;
      }
    }
    const int flag = code != 0;
    const unsigned long long bal = __ballot(flag);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      off += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    if (flag) tile_list[row_base + total + off + pre] = kt;
    total += tot;
    __syncthreads();
  }
  if (tid == 0) tile_cnt[(size_t)t * nqt + qt] = total;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status gsa_build_layout(const gsa_layout* layout, int32_t seq_len, int32_t q_begin,
                                       int32_t q_len, int32_t block_m, int32_t block_n,
                                       const int32_t* sel, const int32_t* sel_groups,
                                       int32_t n_tables, int8_t* table, int32_t* tile_cnt,
                                       int32_t* tile_list, void* stream) {
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  if (block_m < 1 || block_m > 4096) return fail(GSA_EINVAL, "block_m %d outside [1, 4096]", block_m);
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if (n_tables < 1) return fail(GSA_EINVAL, "n_tables %d < 1", n_tables);
  const bool fixed = l.k == 0 && l.G2 == 0;
  if (fixed && (sel || sel_groups)) return fail(GSA_EINVAL, "sel given for the fixed layout");
  if (!fixed && !sel) return fail(GSA_EINVAL, "sel is required when top_k > 0");
  if (l.G2 > 0 && !sel_groups) return fail(GSA_EINVAL, "sel_groups is required with two levels");
  if (l.G2 == 0 && sel_groups) return fail(GSA_EINVAL, "sel_groups given for a single level");
  if (l.k > 64 || l.k2 > 64) return fail(GSA_EUNSUPPORTED, "top_k and l2_top_k are limited to 64");
  if (!table || !tile_cnt || !tile_list) return fail(GSA_EINVAL, "output pointer is NULL");
  const int nqt = (q_len + block_m - 1) / block_m;
  const size_t shm = (size_t)block_m * (sizeof(int) * 6 + sizeof(int) * (l.k + l.k2));
  if (shm > 64 * 1024) return fail(GSA_EUNSUPPORTED, "block_m %d too large for the selection sizes", block_m);
  hipLaunchKernelGGL(k_build_table, dim3(nqt, n_tables), dim3(kThreads), shm,
                     (hipStream_t)stream, l, q_begin, q_len, block_m, nqt, sel, sel_groups, table,
                     tile_cnt, tile_list);
  return launch_status("gsa_build_layout");
}
