"""Seeded synthetic inputs for gist-token sparse attention.

This module only draws random numbers and places them; it holds none of the
method's arithmetic (no scoring, selection, masking or attention).  Both the
oracle-side tests and the HIP path consume exactly these arrays.

Recipe (stated once, used everywhere):
  * ``numpy.random.default_rng(seed)``; draw order Q, then K, then V, each as
    ``standard_normal(float32)`` in C order of its layout, then the plants.
  * bf16 workloads are rounded to bf16 with round-to-nearest-even; the arrays
    stay float32 but hold bf16-representable values, so bf16 -> fp64 is exact.
  * Prefill layout: q ``[B, L, Hq, d]``, k/v ``[B, L, Hkv, d]``.
  * Decode layout: q ``[B, Hq, d]``, k/v cache ``[B, Hkv, kv_len, d]``.
  * Planting (selective decode): the same chunk ids for every KV head of a
    sequence; the gist key of a planted chunk becomes ``0.5 * qbar + N(0,1)``
    where ``qbar`` is the mean of that KV group's query heads.  Two levels:
    planted groups get their level-2 gist keys set that way, then planted
    chunks are drawn from inside the planted groups and get their level-1
    gist keys set that way.
  * Byte sequences (gzip block masks): ``mixed_bytes`` -- per block a kind
    drawn first (0.3 uniform random bytes, 0.5 pseudo-text, 0.2 a short
    repeated pattern), then the contents block by block.  Pseudo-text is
    words of a seeded 24-word vocabulary (2-7 lowercase letters) joined by
    spaces, so blocks range from incompressible to highly compressible.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(a)
    flat_in = a.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        b = flat_in[s:s + step].astype(np.uint64)
        lsb = (b >> np.uint64(16)) & np.uint64(1)
        r = (b + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
        flat_out[s:s + step] = r.astype(np.uint32)
    return out


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def random_qkv(batch, seq_len, hq, hkv, d, seed, dtype="bf16", q_scale=1.0):
    """Q, K, V ~ N(0,1) in prefill layout; ``q_scale`` sharpens the softmax."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(size=(batch, seq_len, hq, d), dtype=np.float32)
    if q_scale != 1.0:
        q = q * np.float32(q_scale)
    k = rng.standard_normal(size=(batch, seq_len, hkv, d), dtype=np.float32)
    v = rng.standard_normal(size=(batch, seq_len, hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def ternary_qkv(batch, seq_len, hq, hkv, d, seed):
    """Small-integer Q, K, V in {-1, 0, 1}: dot products are exact integers in
    any precision, so equal scores really tie."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, size=(batch, seq_len, hq, d)).astype(np.float32)
    k = rng.integers(-1, 2, size=(batch, seq_len, hkv, d)).astype(np.float32)
    v = rng.integers(-1, 2, size=(batch, seq_len, hkv, d)).astype(np.float32)
    return q, k, v


def prefill_inputs(w, seed):
    """Inputs of a prefill workload (see ``workloads.configs``)."""
    return random_qkv(w.batch, w.seq_len, w.hq, w.hkv, w.d, seed, w.dtype)


def _qbar(q, b, h, group):
    # mean of the KV group's query heads; input recipe only
    return q[b, h * group:(h + 1) * group, :].astype(np.float64).mean(axis=0)


def decode_inputs(w, seed):
    """Inputs of a decode workload, with planted gist keys.

    Returns a dict with ``q [B,Hq,d]``, ``k``/``v`` ``[B,Hkv,kv_len,d]`` and the
    planted ids (``plant_chunks [B, n]``, ``plant_groups [B, n2]``).  The
    position of a chunk's or group's gist is where the interleaved layout puts
    it: sinks first, then each chunk's raw tokens followed by its gists (and,
    with two levels, each group's chunks followed by its level-2 gists).
    """
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, L = w.batch, w.hq, w.hkv, w.d, w.seq_len
    G = Hq // Hkv
    q = _normal(rng, (B, Hq, d), w.dtype)
    k = _normal(rng, (B, Hkv, L, d), w.dtype)
    v = _normal(rng, (B, Hkv, L, d), w.dtype)
    S, c, g, P = w.n_sink, w.chunk_len, w.gists, w.period
    out = dict(q=q, k=k, v=v)

    def plant(b, positions):
        for h in range(Hkv):
            qb = _qbar(q, b, h, G)
            for p in positions:
                noise = rng.standard_normal(size=d, dtype=np.float32)
                val = (0.5 * qb + noise).astype(np.float32)
                k[b, h, p, :] = round_bf16(val) if w.dtype == "bf16" else val

    if not w.hierarchical:
        ids = np.zeros((B, w.plant_chunks), dtype=np.int64)
        for b in range(B):
            ids[b] = np.sort(rng.choice(w.n_chunks, size=w.plant_chunks, replace=False))
            plant(b, [S + m * P + c + t for m in ids[b] for t in range(g)])
        out["plant_chunks"] = ids
    else:
        G2, g2, P2 = w.l2_chunks, w.l2_gists, w.group_period
        gids = np.zeros((B, w.plant_groups), dtype=np.int64)
        cids = np.zeros((B, w.plant_chunks), dtype=np.int64)
        for b in range(B):
            gids[b] = np.sort(rng.choice(w.n_groups, size=w.plant_groups, replace=False))
            plant(b, [S + gr * P2 + G2 * P + t for gr in gids[b] for t in range(g2)])
            pool = np.array([gr * G2 + j for gr in gids[b] for j in range(G2)])
            cids[b] = np.sort(rng.choice(pool, size=w.plant_chunks, replace=False))
            pos = []
            for m in cids[b]:
                gr, j = divmod(int(m), G2)
                pos += [S + gr * P2 + j * P + c + t for t in range(g)]
            plant(b, pos)
        out["plant_groups"] = gids
        out["plant_chunks"] = cids
    return out


def mixed_bytes(batch: int, n_bytes: int, block: int, seed: int) -> np.ndarray:
    """uint8 ``[batch, n_bytes]`` with blocks of mixed compressibility."""
    rng = np.random.default_rng(seed)
    nb = -(-n_bytes // block)
    kinds = rng.choice(3, size=(batch, nb), p=[0.3, 0.5, 0.2])
    letters = np.frombuffer(b"abcdefghijklmnopqrstuvwxyz", dtype=np.uint8)
    vocab = [letters[rng.integers(0, 26, int(rng.integers(2, 8)))].tobytes() for _ in range(24)]
    out = np.empty((batch, nb * block), dtype=np.uint8)
    for b in range(batch):
        for i in range(nb):
            if kinds[b, i] == 0:
                blk = rng.integers(0, 256, block, dtype=np.uint8).tobytes()
            elif kinds[b, i] == 1:
                words = []
                while sum(len(w) + 1 for w in words) <= block:
                    words.append(vocab[int(rng.integers(0, len(vocab)))])
                blk = b" ".join(words)[:block]
            else:
                pat = rng.integers(0, 256, int(rng.integers(2, 9)), dtype=np.uint8).tobytes()
                blk = (pat * (block // len(pat) + 1))[:block]
            out[b, i * block:(i + 1) * block] = np.frombuffer(blk, dtype=np.uint8)
    return np.ascontiguousarray(out[:, :n_bytes])
