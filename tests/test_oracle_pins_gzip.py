"""Pins of the gzip-mask oracle (oracle/gzip_mask.py) against facts that do
not come from the oracle itself: a hand-worked example, the causal and band
special cases (closed forms and PyTorch's own attention), a combinatorial edge
count, the flag threshold, and the gzip format's fixed overheads.

Source: Gzip-guided sparse attention page, Core equations.
"""
import json
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import gzip_mask as gm

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    with open(os.path.join(HERE, "golden", "gzip_tiny.json")) as f:
        return json.load(f)


def test_hand_example_flags_mask_and_edges():
    g = _golden()
    x = b"".join(bytes.fromhex(h) for h in g["blocks_hex"])
    r = gm.block_ratios(x, g["block"])
    flags = gm.literal_flags(r)
    assert flags.astype(int).tolist() == g["flags"]
    bm = gm.block_mask(flags, g["w"])
    assert bm.astype(int).tolist() == g["block_mask_lower"]
    tm = gm.token_mask(bm, len(x), g["block"])
    assert gm.edge_count(tm) == g["token_edges"]


def test_flag_threshold_is_strictly_above_the_mean():
    assert gm.literal_flags(np.array([1.0, 2.0, 3.0])).tolist() == [False, False, True]
    assert gm.literal_flags(np.array([0.5, 0.5, 0.5, 0.5])).tolist() == [False] * 4


def test_identical_blocks_have_no_literals():
    x = (b"the same block of bytes, again! " * 2) * 6        # six identical 64-byte blocks
    flags = gm.literal_flags(gm.block_ratios(x, 64))
    assert not flags.any()


def test_short_last_block_is_divided_by_the_block_size():
    # gzip of one byte: a 10-byte header, a fixed-Huffman final block of
    # 3 + 8 + 7 bits (header, the literal, end of block) = 3 bytes, and an
    # 8-byte trailer (RFC 1951 3.2.6, RFC 1952 2.2): 21 bytes in all.
    rng = np.random.default_rng(3)
    x = rng.integers(0, 256, 64, dtype=np.uint8).tobytes() + b"a"
    r = gm.block_ratios(x, 64)
    assert len(r) == 2
    assert r[1] == 21 / 64


@settings(max_examples=40, deadline=None)
@given(nb=st.integers(1, 9), block=st.sampled_from([1, 2, 3, 4]), w=st.integers(0, 4),
       tail=st.integers(0, 3))
def test_no_literals_band_closed_form(nb, block, w, tail):
    L = max(1, (nb - 1) * block + (tail % block if block > 1 else 0) + 1)
    nbl = -(-L // block)
    tm = gm.token_mask(gm.block_mask(np.zeros(nbl, dtype=bool), w), L, block)
    for p in range(L):
        i = p // block
        expect = (i - max(0, i - w)) * block + (p - i * block + 1)
        assert tm[p].sum() == expect
        assert not tm[p, p + 1:].any()


@settings(max_examples=40, deadline=None)
@given(flags=st.lists(st.booleans(), min_size=1, max_size=12), w=st.integers(0, 5))
def test_block_edge_count_combinatorial(flags, w):
    f = np.array(flags, dtype=bool)
    nb = len(f)
    band = sum(min(i, w) + 1 for i in range(nb))
    # literal pairs outside the band: j < i - w, both flagged
    lit_before = np.concatenate([[0], np.cumsum(f)])      # literal blocks among [0, n)
    far = sum(int(lit_before[i - w]) for i in range(nb) if f[i] and i - w > 0)
    assert int(gm.block_mask(f, w).sum()) == band + far


@settings(max_examples=25, deadline=None)
@given(flags=st.lists(st.booleans(), min_size=1, max_size=10), w=st.integers(0, 3))
def test_wide_band_is_causal(flags, w):
    f = np.array(flags, dtype=bool)
    bm = gm.block_mask(f, len(f) - 1 + w)
    assert (bm == np.tril(np.ones((len(f), len(f)), dtype=bool))).all()


def _sdpa(q, k, v, mask=None, causal=False):
    """PyTorch's attention in fp64, KV heads repeated for the query groups."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    am = None if mask is None else torch.from_numpy(mask)[:, None, :, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, is_causal=causal,
                                                         scale=0.3)
    return o.permute(0, 2, 1, 3).numpy()


def test_all_literal_mask_is_causal_attention():
    rng = np.random.default_rng(11)
    B, L, Hq, Hkv, d = 2, 70, 4, 2, 16
    q = rng.standard_normal((B, L, Hq, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    nb = -(-L // 16)
    tm = gm.token_mask(gm.block_mask(np.ones(nb, dtype=bool), 0), L, 16)
    assert (tm == np.tril(np.ones((L, L), dtype=bool))).all()
    o, lse = gm.attend_masked(q, k, v, [tm, tm], 0.3)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)
    # the log-sum-exp of row p over its keys, from its definition
    p, hq = 33, 3
    logits = (k[1, :p + 1, hq // 2, :] @ q[1, p, hq, :]) * 0.3
    assert abs(lse[1, hq, p] - np.log(np.exp(logits).sum())) < 1e-12


def test_gzip_mask_attention_matches_torch_with_the_same_mask():
    rng = np.random.default_rng(12)
    B, L, Hq, Hkv, d, block = 2, 96, 2, 1, 8, 16
    xs = [rng.integers(0, 256, L, dtype=np.uint8).tobytes(), bytes(48) + rng.integers(0, 4, 48, dtype=np.uint8).tobytes()]
    masks = [gm.sequence_mask(x, block, 1) for x in xs]
    q = rng.standard_normal((B, L, Hq, d))
    k = rng.standard_normal((B, L, Hkv, d))
    v = rng.standard_normal((B, L, Hkv, d))
    o, _ = gm.attend_masked(q, k, v, masks, 0.3)
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask=np.stack(masks)), rtol=1e-12, atol=1e-12)


@settings(max_examples=20, deadline=None)
@given(L=st.integers(1, 200), bm=st.sampled_from([4, 8, 16]), bn=st.sampled_from([4, 8]),
       q_begin_t=st.integers(0, 3))
def test_causal_tile_codes_closed_form(L, bm, bn, q_begin_t):
    q_begin = min(L - 1, q_begin_t * bm)
    q_len = L - q_begin
    tm = np.tril(np.ones((L, L), dtype=bool))
    codes = gm.tile_codes(tm, q_begin, q_len, bm, bn)
    for qt in range(codes.shape[0]):
        r0, r1 = q_begin + qt * bm, q_begin + min(q_len, (qt + 1) * bm) - 1
        for t in range(codes.shape[1]):
            c0, c1 = t * bn, min(L, (t + 1) * bn) - 1
            expect = 2 if c1 <= r0 else (0 if c0 > r1 else 1)
            assert codes[qt, t] == expect
