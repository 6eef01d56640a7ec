"""Plain fp64 CPU oracle of gzip-guided block masks.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module; the library path never calls it and it
shares no code with the HIP kernels.

What it computes (Gzip-guided sparse attention page, Core equations):

* The bytes of a sequence are cut into fixed blocks of ``b`` bytes.  Block
  ``i`` gets the compression ratio ``r_i``: the length of its gzip encoding
  (level 1) divided by ``b``; its literal flag is 1 when ``r_i`` is above the
  mean ratio of the sequence's blocks, strictly.
* The block mask joins three parts -- literal-to-literal links (both blocks
  flagged), a local band of blocks at most ``w`` apart, and the diagonal --
  and the result is intersected with the causal mask.  Attention runs over
  byte positions, so token ``p`` sees token ``q`` iff ``q <= p`` and the
  block mask links the block of ``p`` with the block of ``q``.
* Attention is the usual softmax of ``q . k * scale`` over the visible keys,
  every head with the same mask.

Readings where the page leaves a step open:

* The gzip encoding is Python's ``gzip.compress`` at level 1 with a zero
  modification time (the gzip container around zlib's deflate).  A fixed
  header and trailer adds the same amount to every block's length, so the
  flags do not depend on it.
* A short last block (``len(x)`` not a multiple of ``b``) is divided by
  ``b`` as the formula is written, not by its own length.
* ``w`` counts blocks.

Tile codes use the physical key order: tile ``t`` holds key positions
``[t * block_n, (t + 1) * block_n)`` (the last one may be short) and is coded
0 (no visible cell), 2 (all visible) or 1 (otherwise), like the gist
layouts' tables.
"""
import gzip

import numpy as np


def block_ratios(x: bytes, block: int) -> np.ndarray:
    """r_i = |gzip(x[i b : (i + 1) b])| / b for every block of ``x``."""
    nb = -(-len(x) // block)
    return np.array([len(gzip.compress(x[i * block:(i + 1) * block], compresslevel=1, mtime=0)) / block
                     for i in range(nb)], dtype=np.float64)


def literal_flags(r: np.ndarray) -> np.ndarray:
    """1 where a block's ratio is above the mean ratio."""
    return r > r.mean()


def block_mask(flags: np.ndarray, w: int) -> np.ndarray:
    """Boolean [nb, nb]: literal pairs, the band |i - j| <= w, the diagonal;
    causal at block level (a later key block is never visible)."""
    nb = len(flags)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    lit = flags[:, None] & flags[None, :]
    local = np.abs(i - j) <= w
    eye = i == j
    return (lit | local | eye) & (j <= i)


def token_mask(bm: np.ndarray, L: int, block: int) -> np.ndarray:
    """Boolean [L, L]: query p sees key q iff q <= p and the blocks are linked."""
    blk = np.arange(L) // block
    return bm[blk[:, None], blk[None, :]] & (np.arange(L)[None, :] <= np.arange(L)[:, None])


def sequence_mask(x: bytes, block: int, w: int) -> np.ndarray:
    """Token mask of one byte sequence (ratios, flags, block mask, token mask)."""
    return token_mask(block_mask(literal_flags(block_ratios(x, block)), w), len(x), block)


def attend_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, masks, scale: float, rows=None):
    """Masked softmax attention in fp64.

    ``q [B, L, Hq, d]``, ``k``/``v`` ``[B, L, Hkv, d]``, ``masks[b]`` the
    ``[L, L]`` token mask of sequence b.  ``rows`` restricts the work to those
    query positions.  Returns ``o [B, L, Hq, d]`` and ``lse [B, Hq, L]`` (NaN
    where not computed).
    """
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    o = np.full((B, L, Hq, d), np.nan)
    lse = np.full((B, Hq, L), np.nan)
    rows = range(L) if rows is None else rows
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            for p in rows:
                idx = np.nonzero(masks[b][p])[0]
                logits = (k[b, idx, h, :].astype(np.float64) @ q[b, p, hq, :].astype(np.float64)) * scale
                mx = logits.max()
                ls = mx + np.log(np.exp(logits - mx).sum())
                o[b, p, hq, :] = np.exp(logits - ls) @ v[b, idx, h, :].astype(np.float64)
                lse[b, hq, p] = ls
    return o, lse


def tile_codes(mask: np.ndarray, q_begin: int, q_len: int, block_m: int, block_n: int) -> np.ndarray:
    """Codes [nqt, nkt] of one sequence's token mask over query rows
    [q_begin, q_begin + q_len) and key tiles in physical order."""
    L = mask.shape[1]
    nqt = -(-q_len // block_m)
    nkt = -(-L // block_n)
    codes = np.zeros((nqt, nkt), dtype=np.int8)
    for qt in range(nqt):
        r0, r1 = q_begin + qt * block_m, q_begin + min(q_len, (qt + 1) * block_m)
        for t in range(nkt):
            c0, c1 = t * block_n, min(L, (t + 1) * block_n)
            cnt = int(mask[r0:r1, c0:c1].sum())
            codes[qt, t] = 0 if cnt == 0 else (2 if cnt == (r1 - r0) * (c1 - c0) else 1)
    return codes


def edge_count(mask: np.ndarray) -> int:
    """Visible (query, key) pairs of a token mask."""
    return int(mask.sum())
