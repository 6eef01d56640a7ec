// Gzip-guided block masks (Gzip-guided sparse attention page, Core equations):
// per fixed block of bytes a compression ratio and a literal flag, then a
// block mask of literal-to-literal links, a local band of blocks and the
// diagonal, intersected with causality.  The mask reaches the prefill as the
// same kind of tile table the gist layouts use, one table per sequence, with
// key tiles in physical order.
//
//   gsa_gzip_block_flags   host: zlib level-1 gzip of every block, ratios, flags
//   gsa_build_block_mask   device: tile table of the block mask
//   the prefill itself:    gsa_attn_prefill_blockmask (prefill_mfma.hip)
#include <zlib.h>

#include <vector>

#include "gsa_internal.h"

namespace gsa {
namespace {

// One wave per (query tile, sequence).  Every query tile lies inside one
// mask block (block is a multiple of block_m, q_begin of block_m) and every
// key tile inside one (block is a multiple of block_n), so a tile is either
// outside the mask (EMPTY) or takes its causal code: FULL below the diagonal,
// PARTIAL across it, EMPTY above it.
__global__ __launch_bounds__(64) void k_block_mask_table(const int8_t* __restrict__ flags, int nb, int block,
                                                         int w, int L, int q_begin, int q_len, int bm, int bn,
                                                         int nqt, int nkt, int8_t* __restrict__ table,
                                                         int* __restrict__ tile_cnt, int* __restrict__ tile_list) {
  const int qt = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int r0 = q_begin + qt * bm;
  const int r1 = q_begin + imin(q_len, (qt + 1) * bm) - 1;
  const int bi = r0 / block;
  const int8_t* fb = flags + (size_t)b * nb;
  const bool fi = fb[bi] != 0;
  const size_t row = (size_t)b * nqt + qt;
  int count = 0;
  for (int kt0 = 0; kt0 < nkt; kt0 += 64) {
    const int kt = kt0 + lane;
    int code = 0;
    if (kt < nkt) {
      const int c0 = kt * bn, c1 = imin(L, c0 + bn) - 1;
      const int bj = c0 / block;
      const int dist = bi > bj ? bi - bj : bj - bi;
      const bool linked = (fi && fb[bj] != 0) || dist <= w;   // the diagonal is dist 0 <= w
      const int causal = c1 <= r0 ? 2 : (c0 > r1 ? 0 : 1);
      code = linked ? causal : 0;
      table[row * nkt + kt] = (int8_t)code;
    }
    const unsigned long long m = __ballot(code != 0);
    if (code != 0) {
      const int before = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      tile_list[row * nkt + count + before] = kt;
    }
    count += __popcll(m);
  }
  if (lane == 0) tile_cnt[row] = count;
}

}  // namespace
}  // namespace gsa

using namespace gsa;

extern "C" gsa_status gsa_gzip_block_flags(const uint8_t* bytes, int32_t B, int64_t stride_b, int32_t n_bytes,
                                           int32_t block, float* ratio, int8_t* flags) {
  if (!bytes || !flags) return fail(GSA_EINVAL, "bytes or flags is NULL");
  if (B < 1 || n_bytes < 1 || block < 1) return fail(GSA_EINVAL, "B=%d n_bytes=%d block=%d", B, n_bytes, block);
  if (stride_b < n_bytes) return fail(GSA_EINVAL, "stride_b %lld < n_bytes %d", (long long)stride_b, n_bytes);
  const int nb = (n_bytes + block - 1) / block;
  z_stream zs{};
  // level 1, gzip container (window bits 15 + 16), zlib's default memory level
  if (deflateInit2(&zs, 1, Z_DEFLATED, 15 + 16, 8, Z_DEFAULT_STRATEGY) != Z_OK)
    return fail(GSA_EHOST, "zlib deflateInit2 failed");
  std::vector<unsigned char> out(deflateBound(&zs, (uLong)block) + 64);
  std::vector<long long> len(nb);
  gsa_status st = GSA_OK;
  for (int b = 0; b < B && st == GSA_OK; ++b) {
    const uint8_t* x = bytes + (size_t)b * stride_b;
    long long total = 0;
    for (int i = 0; i < nb; ++i) {
      const int n = imin(block, n_bytes - i * block);
      if (deflateReset(&zs) != Z_OK) {
        st = fail(GSA_EHOST, "zlib deflateReset failed");
        break;
      }
      zs.next_in = const_cast<Bytef*>(x + (size_t)i * block);
      zs.avail_in = (uInt)n;
      zs.next_out = out.data();
      zs.avail_out = (uInt)out.size();
      if (deflate(&zs, Z_FINISH) != Z_STREAM_END) {
        st = fail(GSA_EHOST, "zlib deflate did not finish a %d-byte block", n);
        break;
      }
      len[i] = (long long)zs.total_out;
      total += len[i];
    }
    if (st != GSA_OK) break;
    // r_i > mean(r)  <=>  len_i / block > total / (nb * block)  <=>  len_i * nb > total,
    // decided in integers
    for (int i = 0; i < nb; ++i) {
      if (ratio) ratio[(size_t)b * nb + i] = (float)((double)len[i] / (double)block);
      flags[(size_t)b * nb + i] = (int8_t)(len[i] * nb > total);
    }
  }
  deflateEnd(&zs);
  return st;
}

extern "C" gsa_status gsa_build_block_mask(const int8_t* flags, int32_t B, int32_t n_blocks, int32_t block,
                                           int32_t w, int32_t seq_len, int32_t q_begin, int32_t q_len,
                                           int32_t block_m, int32_t block_n, int8_t* table, int32_t* tile_cnt,
                                           int32_t* tile_list, void* stream) {
  if (B < 1 || block < 1 || block_m < 1 || block_n < 1 || w < 0)
    return fail(GSA_EINVAL, "B=%d block=%d block_m=%d block_n=%d w=%d", B, block, block_m, block_n, w);
  if (seq_len < 1 || n_blocks != (seq_len + block - 1) / block)
    return fail(GSA_EINVAL, "n_blocks %d does not cover seq_len %d in blocks of %d", n_blocks, seq_len, block);
  if (block % block_m || block % block_n)
    return fail(GSA_EUNSUPPORTED, "block %d must be a multiple of block_m %d and block_n %d", block, block_m, block_n);
  if (q_begin < 0 || q_len < 0 || q_begin + q_len > seq_len)
    return fail(GSA_EINVAL, "query rows [%d, %d) outside [0, %d)", q_begin, q_begin + q_len, seq_len);
  if (q_begin % block_m) return fail(GSA_EUNSUPPORTED, "q_begin %d is not a multiple of block_m %d", q_begin, block_m);
  if (q_len == 0) return GSA_OK;   // empty query range: no pointer is read
  if (!flags || !table || !tile_cnt || !tile_list) return fail(GSA_EINVAL, "NULL pointer argument");
  const int nqt = (q_len + block_m - 1) / block_m;
  const int nkt = (seq_len + block_n - 1) / block_n;
  hipLaunchKernelGGL(k_block_mask_table, dim3(nqt, B), dim3(64), 0, (hipStream_t)stream, flags, n_blocks, block, w,
                     seq_len, q_begin, q_len, block_m, block_n, nqt, nkt, table, tile_cnt, tile_list);
  return launch_status("gsa_build_block_mask");
}
