"""Pins of the oracle's two-level (gist of gist) branch against rules written
independently of it.

Two-level selection (Forget, Then Recall ... Gist Sparse Attention, abstract:
recursive gist of gist; Simplified Sparse Attention via Gist Tokens, abstract:
H-SSA): a query scores the groups whose level-2 gists all precede it by those
level-2 gist keys and keeps the best l2_top_k; it then scores the chunks of the
kept groups whose gists all precede it by their level-1 gist keys and unfolds
the best top_k.  Ties go to the lower id.

Everything here recomputes that from the modular position classifier of
test_oracle_pins (not from the oracle's type map), with integer-valued inputs
so every score is an exact integer sum, and picks the top-k as the
lexicographically smallest sorted tuple among the subsets of largest total
score (or, for many candidates, by counting the better candidates of each).
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from oracle import gsa_oracle as O
from test_oracle_pins import brute_visible, classify, layouts_2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def best_ids(scores: dict, k: int) -> list:
    """Top-k ids with the lower-id tie rule, from its definition."""
    ids = sorted(scores)
    kk = min(k, len(ids))
    if len(ids) <= 12:
        best = None
        for comb in itertools.combinations(ids, kk):
            key = (-sum(scores[m] for m in comb), comb)
            best = key if best is None or key < best else best
        return list(best[1])
    # an id is chosen iff fewer than k candidates beat it (higher score, or
    # the same score and a lower id)
    return [m for m in ids
            if sum(1 for x in ids if scores[x] > scores[m] or (scores[x] == scores[m] and x < m)) < kk]


def brute_two_level(lay, kinds, qh, kh, i):
    """(kept groups, unfolded chunks) for the query at position i.

    kinds: classify() of every position; qh [G, d], kh [L, d] integer-valued."""
    L = len(kinds)
    l2_gists = {}
    l1_gists = {}
    chunk_group = {}
    for j, (kind, m, grp) in enumerate(kinds):
        if kind == "gist2":
            l2_gists.setdefault(grp, []).append(j)
        elif kind in ("raw", "gist"):
            chunk_group[m] = grp
            if kind == "gist":
                l1_gists.setdefault(m, []).append(j)

    def total(positions):
        return int(sum(int(np.dot(q, kh[j])) for q in qh for j in positions))

    cand_g = [grp for grp, ps in l2_gists.items() if len(ps) == lay.l2_gists and max(ps) < i]
    kept = best_ids({grp: total(l2_gists[grp]) for grp in cand_g}, lay.l2_top_k)
    cand_c = [m for m, ps in l1_gists.items()
              if chunk_group[m] in kept and len(ps) == lay.gists and max(ps) < i]
    sel = best_ids({m: total(l1_gists[m]) for m in cand_c}, lay.top_k)
    assert L == len(kinds)
    return kept, sel


def _pad(ids, k):
    return list(ids) + [-1] * (k - len(ids))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_2, st.integers(0, 10_000), st.integers(1, 3))
def test_two_level_selection_brute_force(case, seed, G):
    """Oracle selection (both levels) equals the brute-force rule on ternary
    inputs, which tie often."""
    lay, L = case
    if L == 0:
        return
    rng = np.random.default_rng(seed)
    d = 3
    q = rng.integers(-1, 2, size=(1, L, G, d)).astype(np.float64)
    k = rng.integers(-1, 2, size=(1, L, 1, d)).astype(np.float64)
    tm = O.type_map(lay, L)
    res = O.select(lay, tm, q, k, list(range(L)), 0.5)
    kinds = [classify(lay, j) for j in range(L)]
    for i in range(L):
        kept, sel = brute_two_level(lay, kinds, q[0, i], k[0, :, 0], i)
        assert res["sel_groups"][0, 0, i].tolist() == _pad(kept, lay.l2_top_k), f"groups at {i}"
        assert res["sel"][0, 0, i].tolist() == _pad(sel, lay.top_k), f"chunks at {i}"


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_2, st.integers(0, 10_000))
def test_two_level_mask_from_brute_selection(case, seed):
    """The oracle's mask rows, given the brute-force selection, equal the
    rule-by-rule predicate (no oracle selection involved)."""
    lay, L = case
    if L == 0:
        return
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, size=(1, L, 2, 3)).astype(np.float64)
    k = rng.integers(-1, 2, size=(1, L, 1, 3)).astype(np.float64)
    tm = O.type_map(lay, L)
    kinds = [classify(lay, j) for j in range(L)]
    for i in range(L):
        kept, sel = brute_two_level(lay, kinds, q[0, i], k[0, :, 0], i)
        row = O.mask_row(lay, tm, i, sel, kept)
        want = [brute_visible(lay, i, j, set(sel), set(kept)) for j in range(L)]
        assert row.tolist() == want


def test_two_level_hand_example():
    """Hand-worked selections and visible set (tests/golden/two_level_tiny.json),
    including queries that sit on a level-2 gist."""
    with open(os.path.join(GOLDEN, "two_level_tiny.json")) as f:
        g = json.load(f)
    L = g["seq_len"]
    d = len(g["q"])
    q = np.tile(np.array(g["q"], dtype=np.float64), (1, L, 1, 1))
    k = np.zeros((1, L, 1, d))
    for pos, key in g["keys"].items():
        k[0, int(pos), 0] = key
    for case in g["queries"]:
        lay = O.Layout.of({**g["layout"], "l2_top_k": case["l2_top_k"]})
        tm = O.type_map(lay, L)
        i = case["i"]
        res = O.select(lay, tm, q[:, i:i + 1], k, [i], 1.0)
        assert res["sel_groups"][0, 0, 0].tolist() == case["sel_groups"], f"groups at {i}"
        assert res["sel"][0, 0, 0].tolist() == case["sel"], f"chunks at {i}"
    lay = O.Layout.of(g["layout"])
    tm = O.type_map(lay, L)
    row = O.mask_row(lay, tm, 11, [2], [1])
    assert np.nonzero(row)[0].tolist() == g["visible_11"]


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(layouts_2, st.integers(1, 5), st.integers(1, 5), st.integers(0, 99))
def test_two_level_block_table_brute_force(case, bm, bn, seed):
    """Two-level tile codes from the rule-by-rule predicate over the stream
    order sinks | level-2 gists | level-1 gists | raws built from the modular
    classifier, with the brute-force selection."""
    lay, L = case
    if L == 0:
        return
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, size=(1, L, 1, 3)).astype(np.float64)
    k = rng.integers(-1, 2, size=(1, L, 1, 3)).astype(np.float64)
    tm = O.type_map(lay, L)
    kinds = [classify(lay, j) for j in range(L)]
    sels, groups = [], []
    for i in range(L):
        kept, sel = brute_two_level(lay, kinds, q[0, i], k[0, :, 0], i)
        sels.append(_pad(sel, lay.top_k))
        groups.append(_pad(kept, lay.l2_top_k))
    tiles = []
    for name in ("sink", "gist2", "gist", "raw"):
        cols = [j for j in range(L) if kinds[j][0] == name]
        tiles += [cols[s:s + bn] for s in range(0, len(cols), bn)]
    codes, vis = O.block_table(lay, tm, 0, L, bm, bn, sels, groups)
    assert codes.shape == (-(-L // bm), len(tiles))
    total = 0
    for qt in range(codes.shape[0]):
        rows = range(qt * bm, min(L, (qt + 1) * bm))
        for t, cols in enumerate(tiles):
            cnt = sum(brute_visible(lay, i, j, set(sels[i]), set(groups[i])) for i in rows for j in cols)
            total += cnt
            want = 0 if cnt == 0 else (2 if cnt == len(rows) * len(cols) else 1)
            assert codes[qt, t] == want
    assert vis == total


def test_two_level_exact_ties_go_to_lower_ids():
    """All level-2 and level-1 gist keys equal: every score ties, so the kept
    groups are the lowest-numbered complete ones and so are the chunks."""
    lay = O.Layout(2, 2, 1, 3, 3, 3, 1, 2)
    P2 = 3 * 3 + 1
    L = 2 + 6 * P2 + 2
    q = np.ones((1, L, 2, 4))
    k = np.ones((1, L, 1, 4))
    tm = O.type_map(lay, L)
    res = O.select(lay, tm, q[:, -1:], k, [L - 1], 0.5)
    assert res["sel_groups"][0, 0, 0].tolist() == [0, 1]
    assert res["sel"][0, 0, 0].tolist() == [0, 1, 2]
