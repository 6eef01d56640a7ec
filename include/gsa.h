/*
 * gsa.h -- C ABI of the gist-token sparse attention library (libgsa.so, gfx950).
 *
 * The method.  A sequence is laid out as n_sink sink tokens, then chunks of
 * chunk_len raw tokens each followed by gists_per_chunk gist tokens (fine,
 * interleaved gists: "A Silver Bullet or a Compromise for Full Attention?",
 * §2 Preliminaries; compression ratio = chunk_len / gists_per_chunk).  A query
 * attends to the sinks, every earlier gist, a causal local window and itself
 * (UniGist summary, Approach), plus the raw tokens of the top_k chunks whose
 * gist keys score highest against it (selective unfolding: Simplified Sparse
 * Attention via Gist Tokens, abstract; Forget, Then Recall ... Gist Sparse
 * Attention, abstract).  top_k = 0 is the fixed sink/gist/window layout.  With
 * l2_chunks > 0 a second level groups l2_chunks chunks followed by l2_gists
 * level-2 gists (gist of gist, same two abstracts): the query scores the
 * groups by their level-2 gists, keeps l2_top_k, scores the chunks of those
 * groups by their level-1 gists and unfolds top_k of them; it sees every
 * level-2 gist, the level-1 gists of the kept groups, the window and the
 * unfolded raw tokens.
 *
 * Readings fixed by this library where the pages are silent: the window W
 * counts interleaved positions and includes the query itself (key j visible
 * iff 0 <= i - j < max(W, 1)); a chunk is a candidate once all its gists are
 * earlier than the query; a chunk's score for one KV head is the mean, over
 * that KV group's query heads (and over the chunk's gists), of q.k*scale; ties
 * go to the lower chunk index.  Q and K arrive after any position encoding.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no device state between calls
 *     (except gsa_attn_decode_noalloc's fixed scratch array, below).
 *   - Work is only enqueued on `stream` (a hipStream_t; NULL = null stream);
 *     no call synchronises.  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Every argument is checked before anything is enqueued: GSA_EINVAL means
 *     nothing was launched; gsa_last_error() gives the reason (thread-local).
 *   - An empty query range (q_len = 0) in the table, selection and prefill
 *     entry points returns GSA_OK once the layout and the range are valid,
 *     without reading any other argument (zero-size tensors may have NULL
 *     pointers).  The backward entry points require q_len >= 1.
 *   - Integer index outputs are int32, ascending, padded with -1.
 *   - Tensors are described by gsa_tensor: element strides for batch, token
 *     position and head; the head dimension d is contiguous.  Pointers must be
 *     16-byte aligned and strides multiples of 16 bytes.
 */
#ifndef GSA_H
#define GSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GSA_OK = 0,
  GSA_EINVAL = 1,        /* bad argument; nothing enqueued */
  GSA_EUNSUPPORTED = 2,  /* valid but not implemented (head dim, dtype, size) */
  GSA_EHIP = 3,          /* the HIP runtime refused a launch */
  GSA_EHOST = 4          /* a host library call (zlib) failed */
} gsa_status;

typedef enum { GSA_F32 = 0, GSA_BF16 = 1 } gsa_dtype;

typedef struct {
  int32_t n_sink;          /* sink tokens at positions [0, n_sink) */
  int32_t chunk_len;       /* c: raw tokens per (level-1) chunk, >= 1 */
  int32_t gists_per_chunk; /* g: gist tokens after each chunk, >= 1 */
  int32_t window;          /* W: local window in positions, self included */
  int32_t top_k;           /* chunks unfolded per query; 0 = fixed layout */
  int32_t l2_chunks;       /* chunks per level-2 group; 0 = single level */
  int32_t l2_gists;        /* level-2 gists after each group */
  int32_t l2_top_k;        /* groups kept per query (two levels) */
} gsa_layout;

typedef struct {
  void* ptr;               /* device pointer to element [0,0,0,0] */
  int32_t dtype;           /* gsa_dtype */
  int32_t reserved;        /* must be 0 */
  int64_t stride_b;        /* elements between batches */
  int64_t stride_t;        /* elements between token positions */
  int64_t stride_h;        /* elements between heads */
} gsa_tensor;

/* Stream-ordered key tiles.  Key columns of the visibility table are the
 * sequence's positions regrouped by stream -- sinks | level-2 gists | gists |
 * raws, ascending inside each stream -- and each stream is cut into tiles of
 * block_n columns (the last tile of a stream may be short; no tile spans two
 * streams).  Rows are query positions [q_begin, q_begin + q_len) cut into
 * tiles of block_m rows.  A tile is coded 0 (no visible pair), 1 (some) or
 * 2 (all).  Grouping the gists into one stream is what lets the prefill skip
 * whole invisible tiles, the purpose UniGist's summary gives for moving its
 * gists (Approach). */

/* Host only.  Table dimensions for a sequence of seq_len positions. */
gsa_status gsa_table_dims(const gsa_layout* layout, int32_t seq_len, int32_t q_len,
                          int32_t block_m, int32_t block_n, int32_t* n_q_tiles,
                          int32_t* n_k_tiles);

/* Block-visibility table (UniGist summary, Approach; SSA abstract for the
 * unfolded chunks).
 *   seq_len       positions of the sequence (keys are [0, seq_len))
 *   q_begin,q_len query rows; q_begin + q_len <= seq_len
 *   sel           NULL iff top_k == 0 and single level; else int32
 *                 [n_tables, q_len, top_k] (the gsa_score_select output of one
 *                 (batch, KV head) per table)
 *   sel_groups    two levels: int32 [n_tables, q_len, l2_top_k]; else NULL
 *   n_tables      1 for the fixed layout, else batch * KV heads
 *   table         int8  [n_tables, n_q_tiles, n_k_tiles]   (out)
 *   tile_cnt      int32 [n_tables, n_q_tiles]              (out) non-empty tiles per row
 *   tile_list     int32 [n_tables, n_q_tiles, n_k_tiles]   (out) their ids, ascending,
 *                 row-padded (entries past tile_cnt are left untouched) */
gsa_status gsa_build_layout(const gsa_layout* layout, int32_t seq_len, int32_t q_begin,
                            int32_t q_len, int32_t block_m, int32_t block_n,
                            const int32_t* sel, const int32_t* sel_groups, int32_t n_tables,
                            int8_t* table, int32_t* tile_cnt, int32_t* tile_list, void* stream);

/* Gist scoring and per-KV-group top-k (SSA abstract: score chunks against the
 * gist keys only, keep the top k; GSA abstract: two levels).
 *   q        [B, q_len, Hq, d] (row r is the query at position q_begin + r)
 *   k        keys of the whole sequence, [B, seq_len, Hkv, d] by strides (a
 *            [B, Hkv, seq_len, d] cache works the same way)
 *   scale    logit scale, normally 1/sqrt(d)
 *   sel      int32 [B, Hkv, q_len, top_k] (out)
 *   sel_groups two levels: int32 [B, Hkv, q_len, l2_top_k] (out); else NULL
 *   scores   nullable float [B, Hkv, q_len, n_cand]: the score of every candidate
 *            of the first level (chunks; groups with two levels), -inf where not
 *            yet a candidate; n_cand = gsa_score_columns().
 * Requires 1 <= top_k <= 64, l2_top_k <= 64, d in {64, 128}. */
gsa_status gsa_score_select(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                            int32_t q_begin, int32_t q_len, float scale, int32_t* sel,
                            int32_t* sel_groups, float* scores, void* stream);

/* Host only.  Columns of the optional scores output of gsa_score_select. */
int32_t gsa_score_columns(const gsa_layout* layout, int32_t seq_len);

/* Block-sparse prefill: softmax attention of every query row over its visible
 * keys -- sinks, every earlier gist and the local window (UniGist summary,
 * Approach), plus the raw tokens of the unfolded chunks (SSA abstract) and,
 * with two levels, the level-1 gists of the kept groups (GSA abstract) --
 * skipping EMPTY tiles and masking only PARTIAL ones (UniGist's summary gives
 * skipping invisible blocks as the aim of moving its gists, Approach).
 *   q, o     [B, q_len, Hq, d]; k, v [B, seq_len, Hkv, d] (by strides)
 *   o        dtype F32, or the input dtype
 *   lse      nullable float [B, Hq, q_len], natural-log log-sum-exp (from an
 *            fp32 sum of the unrounded probabilities; a bf16-input O is
 *            normalised by the sum of the bf16 probabilities it is built from)
 *   sel, sel_groups  as produced by gsa_score_select (NULL for the fixed layout)
 *   table, tile_cnt, tile_list  from gsa_build_layout with the same block_m,
 *            block_n, q_begin, q_len (n_tables = 1 for the fixed layout, else B*Hkv)
 * bf16 with d in {64,128} runs on MFMA and needs block_m, block_n from
 * gsa_prefill_tile(); f32 accepts any block_m and block_n <= 256. */
gsa_status gsa_attn_prefill(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                            gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                            const int32_t* sel, const int32_t* sel_groups, const int8_t* table,
                            const int32_t* tile_cnt, const int32_t* tile_list, int32_t block_m,
                            int32_t block_n, float scale, void* stream);

/* Top-k selection for many query rows at once (SSA abstract: score the
 * chunks against their gist keys only, keep the k best), the same result as
 * gsa_score_select up to fp32 rounding of the scores: per 128 query rows and
 * KV head, one MFMA pass over the gist stream scores every candidate with the
 * sum of the group's query heads split into two bf16 parts (fp32 accuracy;
 * mean and scale are positive factors and do not change the order), and each
 * row keeps its k best by (score desc, chunk index asc), a NaN score ranking
 * as -inf.  Single level with one gist per chunk, bf16, d in {64, 128},
 * 1 <= top_k <= 32, scale > 0 (GSA_EINVAL otherwise).
 *   q    [B, q_len, Hq, d]; k [B, seq_len, Hkv, d] (by strides)
 *   sel  int32 [B, Hkv, q_len, top_k] (out), ascending, -1 padded */
gsa_status gsa_select_prefill(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                              float scale, int32_t* sel, void* stream);

/* Prefill with selective unfolding at scale (SSA abstract; GSA abstract:
 * restore the raw chunks of the selected gists).  A query's visible keys are
 * the fixed part (sinks, earlier gists, window: UniGist summary, Approach)
 * plus the raw tokens of its top_k chosen chunks that lie before its window.
 * The unfolded raws of each (query, KV group) are attended first into a
 * softmax partial per query head (workspace), and the MFMA prefill over the
 * fixed part then starts each row from that partial.
 *   layout  single level, top_k >= 1
 *   sel     int32 [B, Hkv, q_len, top_k]: gsa_select_prefill's (or
 *           gsa_score_select's) output
 *   table, tile_cnt, tile_list  the fixed part's table: gsa_build_layout on
 *           the same layout with top_k = 0, n_tables = 1, the MFMA tile shape
 *   ws      workspace of gsa_prefill_unfolded_workspace_bytes(), 256-byte
 *           aligned (no initialisation needed)
 * bf16 q, k, v; o F32 or BF16; lse nullable [B, Hq, q_len]; d in {64, 128}. */
gsa_status gsa_attn_prefill_unfolded(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                     gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                     int32_t seq_len, int32_t q_begin, int32_t q_len, const int32_t* sel,
                                     const int8_t* table, const int32_t* tile_cnt, const int32_t* tile_list,
                                     int32_t block_m, int32_t block_n, float scale, void* ws, size_t ws_bytes,
                                     void* stream);

/* Host only.  Workspace bytes of gsa_attn_prefill_unfolded. */
size_t gsa_prefill_unfolded_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int32_t q_len);

/* Host only.  Tile shape the prefill kernel for (dtype, d) expects. */
gsa_status gsa_prefill_tile(int32_t dtype, int32_t d, int32_t* block_m, int32_t* block_n);

/* Split-K decode: one query per sequence at position kv_len - 1 (the caller has
 * already appended that token's K and V to the cache), attending to the sinks,
 * every gist earlier than the window (two levels: every level-2 gist and the
 * level-1 gists of the kept groups), the window and the unfolded chunks
 * (decoding with selective unfolding: SSA abstract; gist of gist: GSA
 * abstract; sink + gist + window: UniGist summary, Approach).
 * The log-sum-exp is formed from an fp32 sum of the unrounded probabilities;
 * O is normalised by the sum of the bf16 probabilities it is built from.
 *   q, o     [B, Hq, d] (stride_t unused)
 *   k_cache, v_cache  [B, Hkv, kv_len, d] (by strides), bf16
 *   lse      nullable float [B, Hq]
 *   sel      int32 [B, Hkv, 1, top_k]; sel_groups [B, Hkv, 1, l2_top_k] or NULL
 *   ws       device workspace of at least gsa_decode_workspace_bytes(),
 *            256-byte aligned.  Zero-fill it before its first use: it starts
 *            with per-(batch, KV head) completion counters that every call
 *            leaves at zero again (the partials follow them, so zero it again
 *            before reusing it for a larger batch * KV heads).  Calls that
 *            share one workspace must not overlap (same stream, or serialised
 *            by the caller).
 * Requires bf16 inputs, d in {64,128}, Hq/Hkv <= 16. */
gsa_status gsa_attn_decode(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                           gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B, int32_t Hq,
                           int32_t Hkv, int32_t d, int32_t kv_len, const int32_t* sel,
                           const int32_t* sel_groups, float scale, void* ws, size_t ws_bytes,
                           void* stream);

/* gsa_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * gsa_attn_decode; the completion counters and split partials live in a fixed
 * 8 MiB device array of the library instead (each GPU the library runs on
 * holds its own copy until the process ends).  Limits: batch * KV heads <=
 * 16384, and the split partials of the call must fit the array (GSA_EUNSUPPORTED
 * otherwise, nothing launched).  The first call on a device looks up that
 * device's copy and clears its counters with a fill kernel on `stream`; every
 * call leaves them at zero again.  All calls on one GPU share the array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  Allocates nothing. */
gsa_status gsa_attn_decode_noalloc(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache,
                                   gsa_tensor v_cache, gsa_tensor o, float* lse, int32_t B, int32_t Hq,
                                   int32_t Hkv, int32_t d, int32_t kv_len, const int32_t* sel,
                                   const int32_t* sel_groups, float scale, void* stream);

/* Fused decode step: gsa_score_select followed by gsa_attn_decode for one
 * query per sequence at position kv_len - 1 (selective unfolding: SSA
 * abstract; gist of gist: GSA abstract; sink + gist + window: UniGist summary,
 * Approach), in two kernels that read every visible K/V row from HBM once: the
 * scored gists are visible rows, so their logits give both the scores and the
 * attention.  Results are those of the two separate calls up to fp32 rounding
 * of the scores (a selection can differ only where two candidates' scores
 * are within rounding of each other).
 *   q, o, k_cache, v_cache, lse   as for gsa_attn_decode
 *   sel         int32 [B, Hkv, 1, top_k] (out): the unfolded chunks, ascending,
 *               -1 padded
 *   sel_groups  two levels: int32 [B, Hkv, 1, l2_top_k] (out); else NULL
 *   ws          device workspace of at least gsa_decode_step_workspace_bytes(),
 *               256-byte aligned, zero-filled before its first use (it starts
 *               with per-(batch, KV head) counters that every call leaves at
 *               zero; zero it again before reusing it for a larger
 *               batch * KV heads).  Calls sharing a workspace must not overlap.
 * Requires bf16 inputs, d in {64, 128}, Hq/Hkv <= 16, 1 <= top_k <= 64,
 * l2_top_k <= 64 and l2_top_k * l2_chunks * gists_per_chunk <= 1024. */
gsa_status gsa_decode_step(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache, gsa_tensor v_cache,
                           gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                           int32_t kv_len, float scale, int32_t* sel, int32_t* sel_groups, void* ws,
                           size_t ws_bytes, void* stream);

/* Host only.  Workspace bytes gsa_decode_step needs for these sizes (0 if the
 * sizes are invalid). */
size_t gsa_decode_step_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t d, int32_t kv_len);

/* ---- Compact cache: fixed-layout decode with real KV removal.
 * With the fixed layout (top_k = 0, one level) a query sees only the sinks,
 * every gist and its window (UniGist summary, Approach), so raw tokens that
 * have left the window can be removed from the cache (UniGist summary:
 * removal of the compressed tokens at inference; the Study page, §2
 * Preliminaries: 75% of the KV memory saved at ratio 4).  A compact cache of
 * one (batch, KV head) has gsa_compact_slots() rows:
 *   [ n_sink sink slots | gist_capacity gist slots | W ring slots ]
 * (W = max(window, 1)); the t-th gist of the sequence lives in gist slot t, a
 * raw token at position p in ring slot p mod W.  Caches are [B, Hkv, slots, d]
 * bf16 by strides; other layouts return GSA_EUNSUPPORTED. */

/* Host only.  Rows of a compact cache with room for gist_capacity gists. */
int32_t gsa_compact_slots(const gsa_layout* layout, int32_t gist_capacity);

/* Host only.  Gists among the first seq_len positions (the capacity needed). */
int32_t gsa_compact_gists(const gsa_layout* layout, int32_t seq_len);

/* Writes the K/V of the tokens at positions [pos0, pos0 + n) -- k_new, v_new
 * [B, n, Hkv, d] by strides -- into their slots of the compact caches.  Raw
 * tokens more than W positions before the last one are skipped (no later
 * query can see them).  Positions must be appended in order, each once. */
gsa_status gsa_compact_append(const gsa_layout* layout, gsa_tensor k_new, gsa_tensor v_new, int32_t B,
                              int32_t Hkv, int32_t d, int32_t pos0, int32_t n, gsa_tensor k_cache,
                              gsa_tensor v_cache, int32_t gist_capacity, void* stream);

/* Decode of one query per sequence at position `pos` (its own K/V already
 * appended) over compact caches: softmax attention to the sinks, the gists at
 * or before pos and the raw tokens of its window -- the fixed layout's
 * visible set -- split over many workgroups per (batch, KV head), merged by
 * the last one.  q, o [B, Hq, d]; lse nullable float [B, Hq]; ws a workspace
 * of gsa_compact_decode_workspace_bytes(), 256-byte aligned, zero-filled
 * before first use (its counters are left at zero by every call).
 * Requires bf16 q and caches, d in {64, 128}, Hq/Hkv <= 16. */
gsa_status gsa_compact_decode(const gsa_layout* layout, gsa_tensor q, gsa_tensor k_cache, gsa_tensor v_cache,
                              gsa_tensor o, float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                              int32_t pos, int32_t gist_capacity, float scale, void* ws, size_t ws_bytes,
                              void* stream);

/* Host only.  Workspace bytes gsa_compact_decode needs (0 if invalid). */
size_t gsa_compact_decode_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t d, int32_t pos);

/* Host only.  Workspace bytes gsa_attn_decode needs for these sizes. */
size_t gsa_decode_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t d, int32_t kv_len);

/* ---- Gzip-guided block masks (Gzip-guided sparse attention page, Core
 * equations).  A sequence of bytes is cut into blocks of `block` bytes; block
 * i's ratio is the length of its gzip encoding (zlib, level 1) over `block`,
 * and its literal flag is 1 iff that ratio is above the mean of the
 * sequence's ratios.  Query byte p sees key byte q iff q <= p and the blocks
 * of p and q are linked: both flagged, or at most w blocks apart (which
 * includes the diagonal).  Every head uses the same mask. */

/* Host only: HOST pointers.  bytes [B, n_bytes] with row stride stride_b;
 * ratio (nullable) float [B, n_blocks] and flags int8 [B, n_blocks] (out),
 * n_blocks = ceil(n_bytes / block).  A short last block is divided by
 * `block` too.  The flag compares integer lengths (len_i * n_blocks >
 * sum of lengths), so it is exact.  GSA_EHOST if zlib fails. */
gsa_status gsa_gzip_block_flags(const uint8_t* bytes, int32_t B, int64_t stride_b, int32_t n_bytes,
                                int32_t block, float* ratio, int8_t* flags);

/* Tile table of the block mask, one per sequence, key tiles in physical order
 * (tile t = key bytes [t block_n, (t + 1) block_n), the last may be short):
 * 0 no visible pair, 1 some (the causal diagonal), 2 all.
 *   flags     device int8 [B, n_blocks], n_blocks = ceil(seq_len / block)
 *   table     int8  [B, n_q_tiles, n_k_tiles] (out), n_k_tiles = ceil(seq_len / block_n)
 *   tile_cnt  int32 [B, n_q_tiles] (out); tile_list int32 [B, n_q_tiles, n_k_tiles]
 *             (out, ascending, row-padded as gsa_build_layout's)
 * Requires w >= 0, block a multiple of block_m and of block_n, q_begin a
 * multiple of block_m (a query tile then lies inside one block), else
 * GSA_EUNSUPPORTED. */
gsa_status gsa_build_block_mask(const int8_t* flags, int32_t B, int32_t n_blocks, int32_t block, int32_t w,
                                int32_t seq_len, int32_t q_begin, int32_t q_len, int32_t block_m,
                                int32_t block_n, int8_t* table, int32_t* tile_cnt, int32_t* tile_list,
                                void* stream);

/* Prefill under a block mask: softmax attention of every query row over the
 * keys the table of gsa_build_block_mask (same block_m, block_n, q_begin,
 * q_len) leaves visible, skipping EMPTY tiles and masking PARTIAL ones
 * causally.  q, o [B, q_len, Hq, d]; k, v [B, seq_len, Hkv, d] (by strides);
 * lse nullable float [B, Hq, q_len].  Tile shapes and dtypes as for
 * gsa_attn_prefill (bf16, d in {64, 128} on MFMA with gsa_prefill_tile()). */
gsa_status gsa_attn_prefill_blockmask(gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o, float* lse,
                                      int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                                      int32_t q_begin, int32_t q_len, const int8_t* table,
                                      const int32_t* tile_cnt, const int32_t* tile_list, int32_t block_m,
                                      int32_t block_n, float scale, void* stream);

/* ---- Backward of the block-sparse prefill (Forget, Then Recall ... Gist
 * Sparse Attention, abstract: the sparse pattern is trained end to end; the
 * UniGist summary measures forward and backward latency, Experimental setup).
 * With s = scale q.k, P the softmax over each row's visible keys and
 * D = rowsum(dO * O):  dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T dO, keys summed over the query heads of their KV group.  P is
 * recomputed from the forward's log-sum-exp.
 *   q, do, o, dq  [B, q_len, Hq, d] (by strides); k, v, dk, dv [B, seq_len, Hkv, d]
 *   q, k, v, do   bf16; o F32 or bf16 (the forward's output); dq, dk, dv F32
 *                 or bf16 (all three alike)
 *   lse           float [B, Hq, q_len], natural log, from the forward
 *   sel, sel_groups  the forward's selections (as for gsa_attn_prefill): NULL
 *                 for the fixed layout; sel for top_k > 0; sel_groups too with
 *                 two levels (GSA_EINVAL when they do not match the layout)
 *   table, tile_cnt, tile_list  the forward's tables (gsa_prefill_tile() shape;
 *                 n_tables = 1 for the fixed layout, else B*Hkv)
 *   ws            gsa_prefill_backward_workspace_bytes() bytes (D and the base-2
 *                 log-sum-exp per row are kept there between the two kernels)
 * Every key position of dk and dv is written (zero where no query row sees it).
 * Requires d in {64, 128}.  Any layout; where visibility depends on the
 * selection, PARTIAL tiles test each key against the query's chosen chunks
 * (and groups), as the forward does. */
size_t gsa_prefill_backward_workspace_bytes(int32_t B, int32_t Hq, int32_t q_len);
gsa_status gsa_attn_prefill_backward(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                     gsa_tensor o, gsa_tensor dO, const float* lse, gsa_tensor dq, gsa_tensor dk,
                                     gsa_tensor dv, int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t seq_len,
                                     int32_t q_begin, int32_t q_len, const int32_t* sel, const int32_t* sel_groups,
                                     const int8_t* table, const int32_t* tile_cnt, const int32_t* tile_list,
                                     int32_t block_m, int32_t block_n, float scale, void* ws, size_t ws_bytes,
                                     void* stream);

/* The same backward under a gzip-guided block mask: tables from
 * gsa_build_block_mask (Gzip-guided sparse attention page, Core equations). */
gsa_status gsa_attn_prefill_blockmask_backward(gsa_tensor q, gsa_tensor k, gsa_tensor v, gsa_tensor o,
                                               gsa_tensor dO, const float* lse, gsa_tensor dq, gsa_tensor dk,
                                               gsa_tensor dv, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                               int32_t seq_len, int32_t q_begin, int32_t q_len, const int8_t* table,
                                               const int32_t* tile_cnt, const int32_t* tile_list, int32_t block_m,
                                               int32_t block_n, float scale, void* ws, size_t ws_bytes,
                                               void* stream);

/* The backward of gsa_attn_prefill_unfolded (selective unfolding at scale:
 * SSA abstract; GSA abstract, trained end to end).  A query's keys split into
 * the fixed part and its unfolded raws, disjoint, so: the fixed part's
 * gradients come from the fixed layout's tables as in gsa_attn_prefill_backward,
 * then the unfolded keys add theirs -- to dq from each query's gathered raws,
 * to dk and dv per chunk over the query rows that unfolded it (a per-chunk
 * list in the workspace, walked in ascending row order).  P is recomputed
 * from the forward's log-sum-exp over the union.
 *   layout   single level, top_k >= 1; sel as given to the forward
 *   table, tile_cnt, tile_list  the fixed layout's tables (top_k = 0), as
 *            gsa_attn_prefill_unfolded takes them
 *   o, lse   the unfolded forward's output and log-sum-exp
 *   other arguments and dtypes as gsa_attn_prefill_backward; chunk_len <= 16
 *   ws       gsa_prefill_unfolded_backward_workspace_bytes() bytes, 256-byte
 *            aligned (D, the base-2 lse and the per-chunk lists) */
size_t gsa_prefill_unfolded_backward_workspace_bytes(const gsa_layout* layout, int32_t B, int32_t Hq, int32_t Hkv,
                                                     int32_t seq_len, int32_t q_len);
gsa_status gsa_attn_prefill_unfolded_backward(const gsa_layout* layout, gsa_tensor q, gsa_tensor k, gsa_tensor v,
                                              gsa_tensor o, gsa_tensor dO, const float* lse, gsa_tensor dq,
                                              gsa_tensor dk, gsa_tensor dv, int32_t B, int32_t Hq, int32_t Hkv,
                                              int32_t d, int32_t seq_len, int32_t q_begin, int32_t q_len,
                                              const int32_t* sel, const int8_t* table, const int32_t* tile_cnt,
                                              const int32_t* tile_list, int32_t block_m, int32_t block_n, float scale,
                                              void* ws, size_t ws_bytes, void* stream);

const char* gsa_status_str(gsa_status status);

/* Message of the last non-OK return on the calling thread ("" if none). */
const char* gsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GSA_H */
