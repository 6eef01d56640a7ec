"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form derived from the layout
definition, an independent brute-force rule, a library routine the method
reduces to, or a hand-worked example.  None of them re-types the oracle's own
code.  Layout and visibility rules: UniGist summary (Approach), Simplified
Sparse Attention via Gist Tokens (abstract), Forget, Then Recall ... Gist
Sparse Attention (abstract), Study page "A Silver Bullet or a Compromise for
Full Attention?" (§2 Preliminaries).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import gsa_oracle as O
from workloads import configs, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def classify(lay, j):
    """Independent position classifier by modular arithmetic.

    Returns (kind, chunk, group) with kind in 'sink', 'raw', 'gist', 'gist2'."""
    S, c, g = lay.n_sink, lay.chunk_len, lay.gists
    P = c + g
    if j < S:
        return "sink", -1, -1
    y = j - S
    if not lay.hierarchical:
        m, r = divmod(y, P)
        return ("raw" if r < c else "gist"), m, -1
    G2, g2 = lay.l2_chunks, lay.l2_gists
    P2 = G2 * P + g2
    grp, r2 = divmod(y, P2)
    if r2 >= G2 * P:
        return "gist2", -1, grp
    jj, r = divmod(r2, P)
    return ("raw" if r < c else "gist"), grp * G2 + jj, grp


def brute_visible(lay, i, j, sel=(), selg=()):
    """Rule-by-rule visibility of key j for query i."""
    if j > i:
        return False
    kind, m, grp = classify(lay, j)
    if kind == "sink":
        return True
    if kind == "gist" and not lay.hierarchical:
        return True
    if kind == "gist2":
        return True
    if kind == "gist" and grp in selg:
        return True
    if i - j < max(lay.window, 1):
        return True
    if kind == "raw" and m in sel:
        return True
    return False


def gcnt(lay, x):
    """Closed form: gists at positions < x (single level, unbounded chunks)."""
    S, c, g = lay.n_sink, lay.chunk_len, lay.gists
    P = c + g
    y = max(0, x - S)
    f, r = divmod(y, P)
    return g * f + max(0, r - c)


def closed_visible(lay, i, sel=()):
    """Closed form of |V(i)| for one level."""
    S, c, g = lay.n_sink, lay.chunk_len, lay.gists
    P = c + g
    lo = max(0, i - max(lay.window, 1) + 1)
    n = (i - lo + 1) + min(S, lo) + gcnt(lay, lo)
    for m in sel:
        if m >= 0:
            n += min(max(lo - (S + m * P), 0), c)
    return n


def closed_visible_hier(lay, i, sel=(), selg=()):
    """Closed form of |V(i)| for two levels."""
    S, c, g = lay.n_sink, lay.chunk_len, lay.gists
    P = c + g
    G2, g2 = lay.l2_chunks, lay.l2_gists
    P2 = G2 * P + g2
    lo = max(0, i - max(lay.window, 1) + 1)
    y = max(0, lo - S)
    f, r = divmod(y, P2)
    n = (i - lo + 1) + min(S, lo) + g2 * f + max(0, r - G2 * P)
    for grp in selg:
        if grp < 0:
            continue
        for jj in range(G2):
            n += min(max(lo - (S + grp * P2 + jj * P + c), 0), g)
    for m in sel:
        if m < 0:
            continue
        grp, jj = divmod(m, G2)
        n += min(max(lo - (S + grp * P2 + jj * P), 0), c)
    return n


layouts_1 = st.builds(
    lambda S, c, g, n, W, k, extra: (O.Layout(S, c, g, W, k), S + n * (c + g) + extra),
    st.integers(0, 6), st.integers(1, 6), st.integers(1, 3), st.integers(0, 8),
    st.integers(0, 20), st.integers(0, 9), st.integers(0, 3))

layouts_2 = st.builds(
    lambda S, c, g, G2, g2, ng, W, k, k2, extra: (
        O.Layout(S, c, g, W, k, G2, g2, k2), S + ng * (G2 * (c + g) + g2) + extra),
    st.integers(0, 4), st.integers(1, 4), st.integers(1, 2), st.integers(1, 4),
    st.integers(1, 2), st.integers(0, 4), st.integers(0, 12), st.integers(0, 6),
    st.integers(0, 4), st.integers(0, 3))


# ---------------------------------------------------------------- layout
@settings(max_examples=60, deadline=None)
@given(layouts_1)
def test_type_map_matches_modular_classifier(case):
    lay, L = case
    tm = O.type_map(lay, L)
    assert tm.typ.shape == (L,)
    names = {O.SINK: "sink", O.RAW: "raw", O.GIST: "gist", O.GIST2: "gist2"}
    for j in range(L):
        kind, m, _ = classify(lay, j)
        assert names[int(tm.typ[j])] == kind
        assert int(tm.chunk[j]) == m


@settings(max_examples=40, deadline=None)
@given(layouts_2)
def test_type_map_matches_modular_classifier_two_levels(case):
    lay, L = case
    tm = O.type_map(lay, L)
    names = {O.SINK: "sink", O.RAW: "raw", O.GIST: "gist", O.GIST2: "gist2"}
    for j in range(L):
        kind, m, grp = classify(lay, j)
        assert names[int(tm.typ[j])] == kind
        assert int(tm.chunk[j]) == m
        assert int(tm.group[j]) == grp


@pytest.mark.parametrize("c,g", [(4, 1), (8, 1), (32, 1), (6, 2)])
def test_compression_ratio_and_kv_saving(c, g):
    """Study page §2: ratio = segment length / gist count; at ratio 4 keeping
    only the gists keeps a quarter of the raw KV (75% saved)."""
    lay = O.Layout(0, c, g, 1, 0)
    tm = O.type_map(lay, 50 * (c + g))
    n_raw = int((tm.typ == O.RAW).sum())
    n_gist = int((tm.typ == O.GIST).sum())
    assert n_raw * g == n_gist * c
    if c // g == 4:
        assert 1 - n_gist / n_raw == pytest.approx(0.75)


def test_workload_positions():
    """Position counts that the workload descriptions fix: 548 positions for the
    tiny workload (4 sinks + 32 chunks of 16 raw + 1 gist)."""
    tiny = configs.TINY_PREFILL_F32
    tm = O.type_map(O.Layout.of(tiny.layout), tiny.seq_len)
    assert tiny.seq_len == 548
    assert int((tm.typ == O.RAW).sum()) == 512
    assert int((tm.typ == O.GIST).sum()) == 32
    for w in (configs.LLAMA3B_K0_PREFILL, configs.LLAMA8B_K0_PREFILL):
        tm = O.type_map(O.Layout.of(w.layout), w.seq_len)
        assert int((tm.typ == O.RAW).sum()) == 32768
    h = configs.HIER_DECODE
    tm = O.type_map(O.Layout.of(h.layout), h.seq_len)
    assert int((tm.typ == O.RAW).sum()) == 65536 + 1
    assert int((tm.typ == O.GIST2).sum()) == 1024


# ---------------------------------------------------------------- candidates / scores
def test_candidates_hand_example():
    # S=1, c=2, g=1: 0 sink | 1 2 raw(0) 3 gist(0) | 4 5 raw(1) 6 gist(1) | 7 ...
    lay = O.Layout(1, 2, 1, 1, 1)
    tm = O.type_map(lay, 9)
    assert O.chunk_candidates(lay, tm, 3) == []      # a gist does not see its chunk as done
    assert O.chunk_candidates(lay, tm, 4) == [0]
    assert O.chunk_candidates(lay, tm, 6) == [0]
    assert O.chunk_candidates(lay, tm, 7) == [0, 1]


def test_score_hand_example():
    """Two query heads [1,0,0,0] and [0,1,0,0], gist key [2,4,0,0], d=4:
    logits 2/2 and 4/2, mean 1.5."""
    q = np.array([[1, 0, 0, 0], [0, 1, 0, 0]], dtype=np.float32)
    k = np.zeros((6, 4), dtype=np.float32)
    k[3] = [2, 4, 0, 0]
    s = O.gist_scores(q, k, [[3]], [0], 1 / math.sqrt(4))
    assert s[0] == pytest.approx(1.5, abs=0)
    # two gists [2,4,0,0] and [0,0,0,0]: mean over gists halves it
    s2 = O.gist_scores(q, k, [[3, 4]], [0], 0.5)
    assert s2[0] == pytest.approx(0.75, abs=0)


def test_score_orthogonal_shift_invariance():
    """Adding a vector orthogonal to the group's mean query to every gist key
    leaves every chunk score unchanged."""
    rng = np.random.default_rng(5)
    d, G = 16, 4
    q = rng.standard_normal((G, d))
    k = rng.standard_normal((40, d))
    qbar = q.mean(0)
    u = rng.standard_normal(d)
    u -= qbar * (u @ qbar) / (qbar @ qbar)
    lists = [[j] for j in range(40)]
    a = O.gist_scores(q, k, lists, list(range(40)), 0.25)
    b = O.gist_scores(q, k + u, lists, list(range(40)), 0.25)
    for m in a:
        assert a[m] == pytest.approx(b[m], abs=1e-12)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=0, max_size=9), st.integers(0, 10))
def test_top_k_equals_subset_enumeration(vals, k):
    """Brute force: among all k-subsets with the largest score sum, the
    lexicographically smallest sorted tuple equals (score desc, id asc) top-k."""
    scores = {m: float(v) for m, v in enumerate(vals)}
    chosen, gap = O.top_k(scores, k)
    kk = min(k, len(vals))
    best = None
    for comb in itertools.combinations(range(len(vals)), kk):
        key = (-sum(vals[m] for m in comb), comb)
        best = key if best is None or key < best else best
    assert tuple(chosen) == best[1]
    srt = sorted(vals, reverse=True)
    if 0 < k < len(vals):
        assert gap == srt[k - 1] - srt[k]
    else:
        assert gap == math.inf


def test_selection_nested_in_k():
    """Sel(k) is a subset of Sel(k+1) for every row."""
    lay0 = O.Layout(2, 4, 1, 3, 0)
    L = 2 + 12 * 5
    q, k, _ = inputs.random_qkv(1, L, 2, 1, 8, seed=3, dtype="f32")
    tm = O.type_map(lay0, L)
    prev = None
    for kk in range(0, 8):
        lay = O.Layout(2, 4, 1, 3, kk)
        sel = O.select(lay, tm, q, k, list(range(L)), 0.3)["sel"]
        if prev is not None:
            for r in range(L):
                a = set(x for x in prev[0, 0, r] if x >= 0)
                b = set(x for x in sel[0, 0, r] if x >= 0)
                assert a <= b
        prev = sel


def test_planted_chunks_are_found():
    """Statistical sanity of the planting recipe: in a reduced selective-decode
    workload most planted chunks land in the top-k (not a parity check)."""
    w = configs.Workload(name="t", kind="decode", dtype="bf16", batch=2, hq=8, hkv=2, d=128,
                         n_sink=8, chunk_len=32, gists=1, window=32, top_k=16, n_chunks=256,
                         plant_chunks=16)
    x = inputs.decode_inputs(w, seed=11)
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q = x["q"][:, None]
    kk = np.ascontiguousarray(x["k"].transpose(0, 2, 1, 3))
    res = O.select(lay, tm, q, kk, [L - 1], 1 / math.sqrt(w.d))
    hits = 0
    for b in range(w.batch):
        for h in range(w.hkv):
            hits += len(set(res["sel"][b, h, 0]) & set(x["plant_chunks"][b]))
    assert hits / (w.batch * w.hkv) >= 6


# ---------------------------------------------------------------- visibility
@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_1, st.integers(0, 1000))
def test_mask_equals_brute_force_and_closed_form(case, seed):
    lay, L = case
    if L == 0:
        return
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 2, 1, 4, seed=seed, dtype="f32")
    sel = O.select(lay, tm, q, k, list(range(L)), 0.5)["sel"][0, 0]
    for i in range(L):
        row = O.mask_row(lay, tm, i, sel[i])
        want = [brute_visible(lay, i, j, set(sel[i])) for j in range(L)]
        assert row.tolist() == want
        assert int(row.sum()) == closed_visible(lay, i, sel[i])


@settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_2, st.integers(0, 1000))
def test_mask_two_levels_brute_force_and_closed_form(case, seed):
    lay, L = case
    if L == 0:
        return
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 2, 1, 4, seed=seed, dtype="f32")
    res = O.select(lay, tm, q, k, list(range(L)), 0.5)
    sel, selg = res["sel"][0, 0], res["sel_groups"][0, 0]
    for i in range(L):
        # level-1 choices come only from chosen groups
        for m in sel[i]:
            if m >= 0:
                assert m // lay.l2_chunks in set(selg[i])
        row = O.mask_row(lay, tm, i, sel[i], selg[i])
        want = [brute_visible(lay, i, j, set(sel[i]), set(selg[i])) for j in range(L)]
        assert row.tolist() == want
        assert int(row.sum()) == closed_visible_hier(lay, i, sel[i], selg[i])


@pytest.mark.parametrize("w", [configs.TINY_PREFILL_F32, configs.LLAMA3B_K0_PREFILL,
                               configs.LLAMA8B_K0_PREFILL])
def test_fixed_layout_edge_counts_closed_form(w):
    """Row sums of the k=0 mask equal the closed form (every row for the tiny
    workload, a stride sample for the 32K ones)."""
    lay = O.Layout.of({**w.layout, "top_k": 0})
    L = w.seq_len
    tm = O.type_map(lay, L)
    rows = range(L) if L < 1000 else list(range(0, L, 211)) + [L - 1]
    for i in rows:
        assert int(O.mask_row(lay, tm, i).sum()) == closed_visible(lay, i)
    if L < 1000:
        assert O.edge_count(lay, tm, range(L)) == sum(closed_visible(lay, i) for i in range(L))


def test_decode_rows_closed_form():
    """The decode query's visible set: sinks + every gist + the window + the
    unfolded chunks, minus overlaps, for both decode workloads."""
    for w in (configs.SELECTIVE_DECODE, configs.HIER_DECODE):
        lay = O.Layout.of(w.layout)
        L = w.seq_len
        tm = O.type_map(lay, L)
        i = L - 1
        rng = np.random.default_rng(0)
        if not w.hierarchical:
            sel = np.sort(rng.choice(w.n_chunks, w.top_k, replace=False))
            n = int(O.mask_row(lay, tm, i, sel).sum())
            assert n == closed_visible(lay, i, sel)
        else:
            selg = np.sort(rng.choice(w.n_groups, w.l2_top_k, replace=False))
            pool = [gr * w.l2_chunks + j for gr in selg for j in range(w.l2_chunks)]
            sel = np.sort(rng.choice(pool, w.top_k, replace=False))
            n = int(O.mask_row(lay, tm, i, sel, selg).sum())
            assert n == closed_visible_hier(lay, i, sel, selg)
            if all(gr < w.n_groups - 2 for gr in selg):
                assert n == 128 + 1024 + 64 + 128 + 128 - 2


# ---------------------------------------------------------------- attention
def _sdpa_causal(q, k, v, scale):
    """Dense causal attention by the library routine (fp64, CPU)."""
    B, L, Hq, d = q.shape
    G = Hq // k.shape[2]
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k.astype(np.float64), G, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v.astype(np.float64), G, axis=2)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("two_levels", [False, True])
def test_full_cover_reduces_to_dense_causal(two_levels):
    """With k covering every chunk (and every group) and the window spanning
    the sequence the mask is plain causal, so the output is dense causal
    attention."""
    if two_levels:
        lay = O.Layout(3, 3, 1, 200, 100, 2, 1, 100)
        L = 3 + 6 * 9 + 4
    else:
        lay = O.Layout(3, 5, 2, 200, 100)
        L = 3 + 9 * 7 + 3
    q, k, v = inputs.random_qkv(2, L, 4, 2, 16, seed=7, dtype="f32")
    tm = O.type_map(lay, L)
    res = O.select(lay, tm, q, k, list(range(L)), 0.25)
    o, _ = O.attend(lay, tm, q, k, v, list(range(L)), 0.25, res["sel"], res.get("sel_groups"))
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, 0.25), rtol=0, atol=1e-12)


def test_full_window_alone_is_causal():
    lay = O.Layout(2, 4, 1, 10_000, 0)
    L = 2 + 10 * 5
    q, k, v = inputs.random_qkv(1, L, 2, 1, 8, seed=9, dtype="f32")
    tm = O.type_map(lay, L)
    o, _ = O.attend(lay, tm, q, k, v, list(range(L)), 0.3)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, 0.3), rtol=0, atol=1e-12)


def test_no_chunks_is_sinks_plus_window():
    """With no chunk in the sequence the pattern is sinks + sliding window."""
    lay = O.Layout(4, 1000, 1, 6, 3)
    L = 40
    q, k, v = inputs.random_qkv(1, L, 1, 1, 8, seed=2, dtype="f32")
    tm = O.type_map(lay, L)
    o, lse = O.attend(lay, tm, q, k, v, list(range(L)), 0.4)
    for i in range(L):
        idx = [j for j in range(L) if j <= i and (j < 4 or i - j < 6)]
        lg = np.array([q[0, i, 0].astype(np.float64) @ k[0, j, 0].astype(np.float64) * 0.4
                       for j in idx])
        p = np.exp(lg - lg.max())
        p /= p.sum()
        want = sum(pp * v[0, j, 0].astype(np.float64) for pp, j in zip(p, idx))
        np.testing.assert_allclose(o[0, i, 0], want, rtol=0, atol=1e-12)
        want_lse = lg.max() + math.log(math.fsum(np.exp(lg - lg.max())))
        assert lse[0, 0, i] == pytest.approx(want_lse, abs=1e-12)


def test_special_cases_exact():
    lay = O.Layout(2, 3, 1, 2, 1)
    L = 2 + 6 * 4
    q, k, v = inputs.random_qkv(1, L, 2, 1, 8, seed=4, dtype="f32")
    tm = O.type_map(lay, L)
    sel = O.select(lay, tm, q, k, list(range(L)), 0.3)["sel"]
    # row 0 sees only itself
    o, lse = O.attend(lay, tm, q[:, :1], k, v, [0], 0.3, sel[:, :, :1])
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    # all keys equal, or scale 0: mean of the visible values
    keq = np.broadcast_to(k[:, :1], k.shape).copy()
    for kk, sc in ((keq, 0.3), (k, 0.0)):
        o, _ = O.attend(lay, tm, q, kk, v, list(range(L)), sc, sel)
        for i in range(L):
            idx = [j for j in range(L) if brute_visible(lay, i, j, set(sel[0, 0, i]))]
            want = np.mean(v[0, idx, 0].astype(np.float64), axis=0)
            np.testing.assert_allclose(o[0, i, 0], want, rtol=0, atol=1e-12)
            np.testing.assert_allclose(o[0, i, 1], want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- block table
def test_block_table_hand_example():
    """Hand-worked table of a tiny fixed layout (stored under tests/golden)."""
    with open(os.path.join(GOLDEN, "block_table_tiny.json")) as f:
        g = json.load(f)
    lay = O.Layout.of(g["layout"])
    tm = O.type_map(lay, g["seq_len"])
    codes, vis = O.block_table(lay, tm, 0, g["seq_len"], g["block_m"], g["block_n"])
    assert codes.tolist() == g["codes"]
    assert vis == g["edges"]
    assert O.edge_count(lay, tm, range(g["seq_len"])) == g["edges"]


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_1, st.integers(1, 5), st.integers(1, 5), st.integers(0, 99))
def test_block_table_brute_force(case, bm, bn, seed):
    """Tile codes from the rule-by-rule predicate over an independently built
    stream order, and visible cells summing to the edge count."""
    lay, L = case
    if L == 0:
        return
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 1, 1, 4, seed=seed, dtype="f32")
    sel = O.select(lay, tm, q, k, list(range(L)), 0.5)["sel"][0, 0]
    kinds = [classify(lay, j)[0] for j in range(L)]
    tiles = []
    for name in ("sink", "gist", "raw"):
        cols = [j for j in range(L) if kinds[j] == name]
        tiles += [cols[s:s + bn] for s in range(0, len(cols), bn)]
    codes, vis = O.block_table(lay, tm, 0, L, bm, bn, sel)
    assert codes.shape == (-(-L // bm), len(tiles))
    for qt in range(codes.shape[0]):
        rows = range(qt * bm, min(L, (qt + 1) * bm))
        for t, cols in enumerate(tiles):
            cnt = sum(brute_visible(lay, i, j, set(sel[i])) for i in rows for j in cols)
            want = 0 if cnt == 0 else (2 if cnt == len(rows) * len(cols) else 1)
            assert codes[qt, t] == want
    assert vis == O.edge_count(lay, tm, range(L), sel)


def test_round_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32) * 7
    ours = inputs.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_selection_uses_only_its_query_group():
    """Query head hq belongs to KV head hq // G: the selection of KV head 1 is
    blind to the query heads of group 0 and follows those of group 1.  Group 1's
    queries all point along e1 and only chunk 2's gist key has an e1 part, so
    chunk 2 must be KV head 1's top-1; group 0 is random noise."""
    lay = O.Layout(1, 3, 1, 1, 1)
    L = 1 + 6 * 4
    tm = O.type_map(lay, L)
    d, Hq, Hkv = 8, 4, 2
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, L, Hkv, d))
    k[..., 1] = 0.0
    k[0, tm.chunk_gists[2][0], 1, 1] = 5.0
    base = rng.standard_normal((1, L, Hq, d))
    base[0, :, 2:4, :] = 0.0
    base[0, :, 2:4, 1] = 3.0
    res = O.select(lay, tm, base, k, [L - 1], 0.5)
    assert res["sel"][0, 1, 0, 0] == 2
    noisy = base.copy()
    noisy[0, :, 0:2, :] = rng.standard_normal((L, 2, d)) * 10
    res2 = O.select(lay, tm, noisy, k, [L - 1], 0.5)
    assert np.array_equal(res["sel"][0, 1], res2["sel"][0, 1])
