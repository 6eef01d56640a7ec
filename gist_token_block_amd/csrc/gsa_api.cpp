// Host-side plumbing of libgsa: error reporting, layout validation, the
// host-only query functions of gsa.h.
#include <stdarg.h>
#include <stdio.h>

#include "gsa_internal.h"

namespace gsa {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
}

gsa_status fail(gsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

gsa_status make_lay(const gsa_layout* p, int L, int bn, Lay* out) {
  if (!p) return fail(GSA_EINVAL, "layout is NULL");
  if (p->n_sink < 0) return fail(GSA_EINVAL, "n_sink %d < 0", p->n_sink);
  if (p->chunk_len < 1) return fail(GSA_EINVAL, "chunk_len %d < 1", p->chunk_len);
  if (p->gists_per_chunk < 1) return fail(GSA_EINVAL, "gists_per_chunk %d < 1", p->gists_per_chunk);
  if (p->window < 0) return fail(GSA_EINVAL, "window %d < 0", p->window);
  if (p->top_k < 0) return fail(GSA_EINVAL, "top_k %d < 0", p->top_k);
  if (p->l2_chunks < 0) return fail(GSA_EINVAL, "l2_chunks %d < 0", p->l2_chunks);
  if (p->l2_chunks > 0) {
    if (p->l2_gists < 1) return fail(GSA_EINVAL, "l2_gists %d < 1 with two levels", p->l2_gists);
    if (p->l2_top_k < 1) return fail(GSA_EINVAL, "l2_top_k %d < 1 with two levels", p->l2_top_k);
    if (p->top_k < 1) return fail(GSA_EINVAL, "top_k must be >= 1 with two levels");
  } else if (p->l2_gists != 0 || p->l2_top_k != 0) {
    return fail(GSA_EINVAL, "l2_gists / l2_top_k set without l2_chunks");
  }
  if (L < 0) return fail(GSA_EINVAL, "sequence length %d < 0", L);
  if (p->chunk_len > (1 << 20) || p->gists_per_chunk > (1 << 20) || p->l2_chunks > (1 << 16) ||
      p->l2_gists > (1 << 20))
    return fail(GSA_EUNSUPPORTED, "layout periods too large");
  if (bn < 1) return fail(GSA_EINVAL, "block_n %d < 1", bn);
  Lay l{};
  l.S = p->n_sink;
  l.c = p->chunk_len;
  l.g = p->gists_per_chunk;
  l.P = l.c + l.g;
  l.W1 = p->window > 1 ? p->window : 1;
  l.k = p->top_k;
  l.G2 = p->l2_chunks;
  l.g2 = p->l2_gists;
  l.k2 = p->l2_top_k;
  l.GP = l.G2 * l.P;
  l.P2 = l.GP + l.g2;
  l.L = L;
  l.bn = bn;
  l.dc = make_fdiv(l.c);
  l.dg = make_fdiv(l.g);
  l.dP = make_fdiv(l.P);
  l.dG2 = make_fdiv(l.G2 > 0 ? l.G2 : 1);
  l.dg2 = make_fdiv(l.g2 > 0 ? l.g2 : 1);
  l.dP2 = make_fdiv(l.P2 > 0 ? l.P2 : 1);
  if (l.G2 == 0) {
    l.nstr = 3;
    l.kind[0] = K_SINK; l.kind[1] = K_GIST; l.kind[2] = K_RAW;
  } else {
    l.nstr = 4;
    l.kind[0] = K_SINK; l.kind[1] = K_GIST2; l.kind[2] = K_GIST; l.kind[3] = K_RAW;
  }
  for (int s = 0; s < l.nstr; ++s) {
    StreamMap m{};
    m.per = 1; m.G = 1 << 30; m.stride1 = 1; m.stride2 = 0; m.base = 0;
    switch (l.kind[s]) {
      case K_SINK: break;
      case K_GIST2: m.per = l.g2; m.stride1 = l.P2; m.base = l.S + l.GP; break;
      case K_GIST:
        m.per = l.g; m.stride1 = l.P; m.base = l.S + l.c;
        if (l.G2) { m.G = l.G2; m.stride2 = l.P2; }
        break;
      case K_RAW:
        m.per = l.c; m.stride1 = l.P; m.base = l.S;
        if (l.G2) { m.G = l.G2; m.stride2 = l.P2; }
        break;
    }
    m.dper = make_fdiv(m.per);
    m.dG = make_fdiv(m.G);
    l.smap[s] = m;
  }
  int t0 = 0;
  for (int s = 0; s < l.nstr; ++s) {
    l.len[s] = count_below(l, l.kind[s], L);
    l.tile0[s] = t0;
    t0 += (l.len[s] + bn - 1) / bn;
  }
  l.nkt = t0;
  for (int s = l.nstr; s < 4; ++s) {
    l.tile0[s] = t0;
    l.len[s] = 0;
    l.kind[s] = K_RAW;
    l.smap[s] = l.smap[l.nstr - 1];
  }
  *out = l;
  return GSA_OK;
}

gsa_status check_tensor(const char* name, const gsa_tensor& t, int d, bool) {
  if (!t.ptr) return fail(GSA_EINVAL, "%s.ptr is NULL", name);
  if (t.dtype != GSA_F32 && t.dtype != GSA_BF16) return fail(GSA_EINVAL, "%s.dtype %d unknown", name, t.dtype);
  if (t.reserved != 0) return fail(GSA_EINVAL, "%s.reserved must be 0", name);
  const int esz = t.dtype == GSA_F32 ? 4 : 2;
  if (reinterpret_cast<uintptr_t>(t.ptr) % 16) return fail(GSA_EINVAL, "%s.ptr not 16-byte aligned", name);
  if ((t.stride_b * esz) % 16 || (t.stride_t * esz) % 16 || (t.stride_h * esz) % 16)
    return fail(GSA_EINVAL, "%s strides must be multiples of 16 bytes", name);
  if (t.stride_b < 0 || t.stride_t < 0 || t.stride_h < 0) return fail(GSA_EINVAL, "%s has a negative stride", name);
  (void)d;
  return GSA_OK;
}

gsa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GSA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return GSA_OK;
}

}  // namespace gsa

using namespace gsa;

extern "C" {

const char* gsa_status_str(gsa_status s) {
  switch (s) {
    case GSA_OK: return "GSA_OK";
    case GSA_EINVAL: return "GSA_EINVAL";
    case GSA_EUNSUPPORTED: return "GSA_EUNSUPPORTED";
    case GSA_EHIP: return "GSA_EHIP";
    case GSA_EHOST: return "GSA_EHOST";
  }
  return "GSA_UNKNOWN";
}

const char* gsa_last_error(void) { return g_err.c_str(); }

gsa_status gsa_table_dims(const gsa_layout* layout, int32_t seq_len, int32_t q_len, int32_t block_m,
                          int32_t block_n, int32_t* nqt, int32_t* nkt) {
  if (!nqt || !nkt) return fail(GSA_EINVAL, "output pointers are NULL");
  if (block_m < 1) return fail(GSA_EINVAL, "block_m %d < 1", block_m);
  if (q_len < 0) return fail(GSA_EINVAL, "q_len %d < 0", q_len);
  Lay l;
  gsa_status st = make_lay(layout, seq_len, block_n, &l);
  if (st != GSA_OK) return st;
  *nqt = (q_len + block_m - 1) / block_m;
  *nkt = l.nkt;
  return GSA_OK;
}

int32_t gsa_score_columns(const gsa_layout* layout, int32_t seq_len) {
  Lay l;
  if (make_lay(layout, seq_len, 1, &l) != GSA_OK) return -1;
  if (l.G2 == 0) return count_below(l, K_GIST, seq_len) / l.g;
  return count_below(l, K_GIST2, seq_len) / l.g2;
}

gsa_status gsa_prefill_tile(int32_t dtype, int32_t d, int32_t* block_m, int32_t* block_n) {
  if (!block_m || !block_n) return fail(GSA_EINVAL, "output pointers are NULL");
  if (dtype == GSA_BF16 && (d == 64 || d == 128)) {
    *block_m = 128;
    *block_n = 64;
    return GSA_OK;
  }
  if (dtype == GSA_F32 || dtype == GSA_BF16) {
    *block_m = 64;
    *block_n = 64;
    return GSA_OK;
  }
  return fail(GSA_EINVAL, "dtype %d unknown", dtype);
}

}  // extern "C"
