"""Plain fp64 CPU oracle of gist-token sparse attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  The library path never calls it, and it
shares no code with the HIP kernels: it builds the sequence position by
position, materialises explicit boolean mask rows and runs textbook softmax
attention in float64 with numpy.

What it computes, and where the pages state it:

* Sequence layout.  Sink tokens first, then chunks of ``c`` raw tokens, each
  followed by ``g`` gist tokens (interleaved, fine-grained gists: Study page
  "A Silver Bullet or a Compromise for Full Attention?", §2 Preliminaries;
  Simplified Sparse Attention via Gist Tokens, abstract; UniGist summary,
  Approach).  The compression ratio is ``c / g`` (Study page, §2).
* Two levels (gist of gist: Forget, Then Recall ... Gist Sparse Attention,
  abstract; the H-SSA variant in the SSA abstract).  A group is ``G2`` level-1
  chunks followed by ``g2`` level-2 gists.
* Selective unfolding (SSA abstract; GSA abstract).  A query scores the chunks
  whose gists are all earlier than it, by attention logits against the gist
  keys only, and unfolds the raw tokens of the top-k chunks.  The score of a
  chunk for one KV head is the mean over that KV group's query heads of
  ``q . k_gist / sqrt(d)``; with ``g > 1`` it is also averaged over the
  chunk's gists.  Ties go to the lower chunk index; the chosen ids are stored
  ascending, padded with -1.
* Visibility (UniGist summary, Approach: sinks, gists and a local window;
  SSA abstract: plus the unfolded raw tokens).  Key ``j`` is visible to query
  ``i`` iff ``j <= i`` and one of: ``j`` is a sink; ``j`` is a gist (single
  level) or a level-2 gist; ``j`` is a level-1 gist of a selected group;
  ``i - j < max(W, 1)``; ``j`` is a raw token of a selected chunk.
* Attention.  Softmax over the visible keys of ``q . k * scale``, fp64,
  returning the output and the log-sum-exp.
* Block table.  Key columns permuted into stream order (sinks | level-2 gists
  | gists | raws), each stream cut into tiles of ``BN`` (the last one may be
  short), query rows cut into tiles of ``BM``; a tile is coded 0 (no visible
  cell), 2 (all visible) or 1 (otherwise).  The stream-ordered view is this
  library's way of letting a kernel skip invisible tiles, the aim UniGist's
  summary gives for moving its gists (Approach).

Parity unpinned: the averaging of a chunk score over ``g > 1`` gists (no page
fixes it, no workload uses it).  Every other function is pinned by the
``-m "not gpu"`` tests (closed forms, brute force, textbook reductions).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SINK, RAW, GIST, GIST2 = 0, 1, 2, 3


@dataclass(frozen=True)
class Layout:
    n_sink: int
    chunk_len: int
    gists: int
    window: int
    top_k: int
    l2_chunks: int = 0
    l2_gists: int = 0
    l2_top_k: int = 0

    @property
    def hierarchical(self) -> bool:
        return self.l2_chunks > 0

    @staticmethod
    def of(d: dict) -> "Layout":
        return Layout(**{k: int(v) for k, v in d.items()})


@dataclass
class TypeMap:
    typ: np.ndarray          # [L] SINK / RAW / GIST / GIST2
    chunk: np.ndarray        # [L] level-1 chunk id of raw and gist tokens, else -1
    group: np.ndarray        # [L] level-2 group id (two levels), else -1
    chunk_gists: list        # chunk id -> list of its gist positions (present ones)
    group_gists: list        # group id -> list of its level-2 gist positions
    chunk_group: list        # chunk id -> group id (two levels) or -1


def type_map(lay: Layout, L: int) -> TypeMap:
    """Build the interleaved sequence token by token, truncated to ``L``."""
    typ, chunk, group = [], [], []
    chunk_gists, group_gists, chunk_group = [], [], []

    def put(t, m, gr):
        if len(typ) < L:
            typ.append(t)
            chunk.append(m)
            group.append(gr)
            return True
        return False

    for _ in range(lay.n_sink):
        put(SINK, -1, -1)
    m = 0
    gr = 0
    while len(typ) < L:
        if not lay.hierarchical:
            chunk_gists.append([])
            chunk_group.append(-1)
            for _ in range(lay.chunk_len):
                put(RAW, m, -1)
            for _ in range(lay.gists):
                if put(GIST, m, -1):
                    chunk_gists[m].append(len(typ) - 1)
            m += 1
        else:
            group_gists.append([])
            for _ in range(lay.l2_chunks):
                chunk_gists.append([])
                chunk_group.append(gr)
                for _ in range(lay.chunk_len):
                    put(RAW, m, gr)
                for _ in range(lay.gists):
                    if put(GIST, m, gr):
                        chunk_gists[m].append(len(typ) - 1)
                m += 1
            for _ in range(lay.l2_gists):
                if put(GIST2, -1, gr):
                    group_gists[gr].append(len(typ) - 1)
            gr += 1
    return TypeMap(np.array(typ, dtype=np.int64), np.array(chunk, dtype=np.int64),
                   np.array(group, dtype=np.int64), chunk_gists, group_gists, chunk_group)


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def chunk_candidates(lay: Layout, tm: TypeMap, i: int) -> list:
    """Level-1 chunks whose gists are all present and all earlier than ``i``."""
    return [m for m, gp in enumerate(tm.chunk_gists)
            if len(gp) == lay.gists and gp[-1] < i]


def group_candidates(lay: Layout, tm: TypeMap, i: int) -> list:
    """Level-2 groups whose level-2 gists are all present and earlier than ``i``."""
    return [gr for gr, gp in enumerate(tm.group_gists)
            if len(gp) == lay.l2_gists and gp[-1] < i]


def gist_scores(q_group: np.ndarray, k_head: np.ndarray, gist_lists: list, ids: list,
                scale: float) -> dict:
    """Score of each id: mean over the query heads (rows of ``q_group``) and over
    the id's gist keys of ``q . k * scale``.  ``k_head`` is ``[L, d]``."""
    qg = q_group.astype(np.float64)
    out = {}
    for m in ids:
        kg = k_head[gist_lists[m], :].astype(np.float64)
        out[m] = float((qg @ kg.T).mean() * scale)
    return out


def top_k(scores: dict, k: int):
    """Best ``k`` ids by (score descending, id ascending).

    Returns (chosen ids ascending, gap) where gap is the k-th best score minus
    the (k+1)-th, or +inf when there are at most k candidates."""
    order = sorted(scores, key=lambda m: (-scores[m], m))
    chosen = sorted(order[:k])
    if k > 0 and len(order) > k:
        gap = scores[order[k - 1]] - scores[order[k]]
    else:
        gap = math.inf
    return chosen, gap


def _pad(ids, k):
    return list(ids) + [-1] * (k - len(ids))


def select(lay: Layout, tm: TypeMap, q: np.ndarray, k: np.ndarray, positions, scale: float,
           forced_groups=None):
    """Per (batch, KV head, query) selection.

    ``q`` is ``[B, Nq, Hq, d]`` (row r sits at ``positions[r]``), ``k`` is
    ``[B, L, Hkv, d]``.  Returns a dict with ``sel [B,Hkv,Nq,k]`` and ``gap``;
    two levels add ``sel_groups [B,Hkv,Nq,k2]`` and ``gap2``.  Level-1
    candidates of the two-level form are the chunks of the chosen groups;
    ``forced_groups`` (same shape as ``sel_groups``) replaces the level-2
    choice, which the comparison protocol uses after a near-tie swap.
    """
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    K1 = lay.top_k
    sel = np.full((B, Hkv, Nq, K1), -1, dtype=np.int64)
    gap = np.full((B, Hkv, Nq), math.inf)
    out = dict(sel=sel, gap=gap)
    if lay.hierarchical:
        K2 = lay.l2_top_k
        selg = np.full((B, Hkv, Nq, K2), -1, dtype=np.int64)
        gap2 = np.full((B, Hkv, Nq), math.inf)
        out.update(sel_groups=selg, gap2=gap2)
    for b in range(B):
        for h in range(Hkv):
            kh = k[b, :, h, :]
            for r, i in enumerate(positions):
                qg = q[b, r, h * G:(h + 1) * G, :]
                if not lay.hierarchical:
                    s = gist_scores(qg, kh, tm.chunk_gists, chunk_candidates(lay, tm, i), scale)
                    ids, gp = top_k(s, K1)
                    sel[b, h, r] = _pad(ids, K1)
                    gap[b, h, r] = gp
                else:
                    if forced_groups is not None:
                        gids = [x for x in forced_groups[b, h, r] if x >= 0]
                        gp2 = math.inf
                    else:
                        s2 = gist_scores(qg, kh, tm.group_gists, group_candidates(lay, tm, i),
                                         scale)
                        gids, gp2 = top_k(s2, K2)
                    selg[b, h, r] = _pad(gids, K2)
                    gap2[b, h, r] = gp2
                    cands = [m for m, gr in enumerate(tm.chunk_group)
                             if gr in gids and len(tm.chunk_gists[m]) == lay.gists
                             and tm.chunk_gists[m][-1] < i]
                    s1 = gist_scores(qg, kh, tm.chunk_gists, cands, scale)
                    ids, gp = top_k(s1, K1)
                    sel[b, h, r] = _pad(ids, K1)
                    gap[b, h, r] = gp
    return out


# --------------------------------------------------------------------------
# visibility, attention, block table
# --------------------------------------------------------------------------

def mask_row(lay: Layout, tm: TypeMap, i: int, sel_ids=(), group_ids=()) -> np.ndarray:
    """Boolean visibility of every key position ``j < L`` for the query at ``i``."""
    L = tm.typ.shape[0]
    j = np.arange(L)
    typ = tm.typ
    sel_ids = [x for x in sel_ids if x >= 0]
    group_ids = [x for x in group_ids if x >= 0]
    vis = typ == SINK
    if lay.hierarchical:
        vis = vis | (typ == GIST2) | ((typ == GIST) & np.isin(tm.group, group_ids))
    else:
        vis = vis | (typ == GIST)
    vis = vis | ((i - j) < max(lay.window, 1))
    vis = vis | ((typ == RAW) & np.isin(tm.chunk, sel_ids))
    return vis & (j <= i)


def _row_sel(sel, b, h, r):
    return () if sel is None else sel[b, h, r]


def attend(lay: Layout, tm: TypeMap, q: np.ndarray, k: np.ndarray, v: np.ndarray, positions,
           scale: float, sel=None, sel_groups=None, rows=None):
    """Masked softmax attention in fp64.

    ``q [B, Nq, Hq, d]`` with row r at ``positions[r]``; ``k``/``v``
    ``[B, L, Hkv, d]``.  ``rows`` restricts the work to those row indices.
    Returns ``o [B, Nq, Hq, d]`` and ``lse [B, Hq, Nq]`` (NaN where not computed).
    """
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    o = np.full((B, Nq, Hq, d), np.nan)
    lse = np.full((B, Hq, Nq), np.nan)
    rows = range(Nq) if rows is None else rows
    for b in range(B):
        for h in range(Hkv):
            for r in rows:
                i = positions[r]
                vis = mask_row(lay, tm, i, _row_sel(sel, b, h, r), _row_sel(sel_groups, b, h, r))
                idx = np.nonzero(vis)[0]
                kk = k[b, idx, h, :].astype(np.float64)
                vv = v[b, idx, h, :].astype(np.float64)
                qq = q[b, r, h * G:(h + 1) * G, :].astype(np.float64)
                logits = (qq @ kk.T) * scale                     # [G, n]
                mx = logits.max(axis=1, keepdims=True)
                ls = mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True))
                p = np.exp(logits - ls)
                o[b, r, h * G:(h + 1) * G, :] = p @ vv
                lse[b, h * G:(h + 1) * G, r] = ls[:, 0]
    return o, lse


def stream_columns(lay: Layout, tm: TypeMap) -> list:
    """Key positions of each stream, in stream order."""
    if lay.hierarchical:
        kinds = [SINK, GIST2, GIST, RAW]
    else:
        kinds = [SINK, GIST, RAW]
    return [np.nonzero(tm.typ == t)[0] for t in kinds]


def column_tiles(lay: Layout, tm: TypeMap, block_n: int) -> list:
    """Position arrays of each key tile: streams cut into ``block_n`` wide pieces."""
    tiles = []
    for pos in stream_columns(lay, tm):
        for s in range(0, len(pos), block_n):
            tiles.append(pos[s:s + block_n])
    return tiles


def block_table(lay: Layout, tm: TypeMap, q_begin: int, q_len: int, block_m: int, block_n: int,
                sel_rows=None, group_rows=None, row_tiles=None):
    """Codes of one visibility table ``[nqt, nkt]`` (0 empty, 1 partial, 2 full).

    ``sel_rows``/``group_rows`` are the selections of the ``q_len`` rows
    (``[q_len, k]``), or None for the fixed layout.  ``row_tiles`` restricts the
    computed query tiles (others stay -1).  Also returns the visible-cell count
    of the computed tiles.
    """
    tiles = column_tiles(lay, tm, block_n)
    nqt = -(-q_len // block_m)
    codes = np.full((nqt, len(tiles)), -1, dtype=np.int8)
    visible = 0
    for qt in (range(nqt) if row_tiles is None else row_tiles):
        r0, r1 = qt * block_m, min(q_len, (qt + 1) * block_m)
        rows = []
        for r in range(r0, r1):
            s = () if sel_rows is None else sel_rows[r]
            gsel = () if group_rows is None else group_rows[r]
            rows.append(mask_row(lay, tm, q_begin + r, s, gsel))
        M = np.stack(rows)
        for t, cols in enumerate(tiles):
            cnt = int(M[:, cols].sum())
            visible += cnt
            codes[qt, t] = 0 if cnt == 0 else (2 if cnt == M.shape[0] * len(cols) else 1)
    return codes, visible


def tile_lists(codes: np.ndarray) -> list:
    """Non-empty tile ids of each query-tile row, ascending."""
    return [np.nonzero(row > 0)[0] for row in codes]


def edge_count(lay: Layout, tm: TypeMap, positions, sel_rows=None, group_rows=None) -> int:
    """Number of visible (query, key) pairs over the given query positions."""
    e = 0
    for r, i in enumerate(positions):
        s = () if sel_rows is None else sel_rows[r]
        gsel = () if group_rows is None else group_rows[r]
        e += int(mask_row(lay, tm, i, s, gsel).sum())
    return e
