"""GPU parity: block-visibility tables and tile lists, bit-exact vs the oracle."""
import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import dev, to_dev

pytestmark = pytest.mark.gpu


def _gpu_table(layout, L, q_begin, q_len, bm, bn, sel=None, selg=None, n_tables=1):
    s = None if sel is None else torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).to(dev())
    g = None if selg is None else torch.from_numpy(np.ascontiguousarray(selg, dtype=np.int32)).to(dev())
    table, cnt, lst = gsa.build_layout(layout, L, q_begin, q_len, bm, bn, s, g, n_tables)
    torch.cuda.synchronize()
    return table.cpu().numpy(), cnt.cpu().numpy(), lst.cpu().numpy()


def _compare(codes_ref, table, cnt, lst, rows=None):
    rows = range(codes_ref.shape[0]) if rows is None else rows
    for qt in rows:
        assert np.array_equal(table[qt], codes_ref[qt]), f"query tile {qt} codes differ"
        want = np.nonzero(codes_ref[qt] > 0)[0]
        assert cnt[qt] == len(want), f"query tile {qt} count"
        assert np.array_equal(lst[qt, :cnt[qt]], want), f"query tile {qt} list"


CASES = [
    # (layout, L, q_begin, q_len, bm, bn)
    (dict(n_sink=2, chunk_len=2, gists=1, window=1, top_k=0), 8, 0, 8, 4, 2),
    (dict(n_sink=5, chunk_len=3, gists=2, window=7, top_k=0), 5 + 40 * 5 + 3, 0, 5 + 40 * 5 + 3, 16, 16),
    (dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0), 128 + 700 * 5, 0, 128 + 700 * 5, 128, 64),
    (dict(n_sink=0, chunk_len=8, gists=1, window=0, top_k=0), 9 * 90 + 4, 37, 500, 64, 64),
    (dict(n_sink=3, chunk_len=6, gists=1, window=10, top_k=3), 3 + 50 * 7 + 2, 0, 3 + 50 * 7 + 2, 32, 16),
    (dict(n_sink=3, chunk_len=4, gists=1, window=6, top_k=3, l2_chunks=3, l2_gists=1, l2_top_k=2),
     3 + 12 * 16 + 5, 0, 3 + 12 * 16 + 5, 16, 8),
    # window of 2 behind 3 gists: query tiles [3,4], [13,14], ... reach a raw
    # tile only through rows whose windows hold no raw at all (EMPTY tiles)
    (dict(n_sink=0, chunk_len=2, gists=3, window=2, top_k=0), 100, 3, 97, 2, 4),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_table_small_layouts(case):
    layout, L, qb, ql, bm, bn = CASES[case]
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    sel = selg = None
    n_tables = 1
    B, Hkv = 2, 2
    if lay.top_k > 0 or lay.hierarchical:
        q, k, _ = inputs.random_qkv(B, L, 2 * Hkv, Hkv, 16, seed=case, dtype="f32")
        res = O.select(lay, tm, q[:, qb:qb + ql], k, list(range(qb, qb + ql)), 0.25)
        sel = res["sel"]
        selg = res.get("sel_groups")
        n_tables = B * Hkv
    table, cnt, lst = _gpu_table(layout, L, qb, ql, bm, bn,
                                 None if sel is None else sel.reshape(n_tables, ql, -1),
                                 None if selg is None else selg.reshape(n_tables, ql, -1), n_tables)
    for t in range(n_tables):
        srow = None if sel is None else sel.reshape(n_tables, ql, -1)[t]
        grow = None if selg is None else selg.reshape(n_tables, ql, -1)[t]
        codes, _ = O.block_table(lay, tm, qb, ql, bm, bn, srow, grow)
        _compare(codes, table[t], cnt[t], lst[t])


@pytest.mark.parametrize("w", [configs.LLAMA3B_K0_PREFILL, configs.LLAMA8B_K0_PREFILL],
                         ids=lambda w: w.name)
def test_table_full_size_fixed_layout(w):
    """Full 32K tables at the prefill kernel's 128x64 tiles; the oracle checks
    a spread of query-tile rows (first, last, a stride sample)."""
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    table, cnt, lst = _gpu_table(w.layout, L, 0, L, 128, 64)
    nqt = table.shape[1]
    rows = sorted(set([0, 1, 2, nqt - 2, nqt - 1] + list(range(3, nqt, 37))))
    codes, _ = O.block_table(lay, tm, 0, L, 128, 64, row_tiles=rows)
    _compare(codes, table[0], cnt[0], lst[0], rows)
    # totals that the closed form fixes: every row's visible cells are counted once
    assert int((table[0] > 0).sum()) == int(cnt[0].sum())


def test_table_tiny_prefill_with_selection():
    w = configs.TINY_PREFILL_F32
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q, k, _ = inputs.prefill_inputs(w, seed=0)
    res = O.select(lay, tm, q, k, list(range(L)), 1 / np.sqrt(w.d))
    for bm, bn in ((64, 64), (16, 16), (128, 64)):
        table, cnt, lst = _gpu_table(w.layout, L, 0, L, bm, bn, res["sel"].reshape(1, L, -1), None, 1)
        codes, vis = O.block_table(lay, tm, 0, L, bm, bn, res["sel"][0, 0])
        _compare(codes, table[0], cnt[0], lst[0])


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
def test_table_decode_row(w):
    """One-row tables of the decode query with random valid selections."""
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    rng = np.random.default_rng(3)
    T = 4
    if w.hierarchical:
        selg = np.stack([np.sort(rng.choice(w.n_groups, w.l2_top_k, replace=False)) for _ in range(T)])
        sel = np.stack([np.sort(rng.choice([g * w.l2_chunks + j for g in selg[t] for j in range(w.l2_chunks)],
                                           w.top_k, replace=False)) for t in range(T)])
        selg[0, -2:] = [w.n_groups - 2, w.n_groups - 1]       # groups touching the window
        selg[0].sort()
    else:
        selg = None
        sel = np.stack([np.sort(rng.choice(w.n_chunks, w.top_k, replace=False)) for _ in range(T)])
        sel[0, -1] = w.n_chunks - 1                              # a chunk inside the window
    table, cnt, lst = _gpu_table(w.layout, L, L - 1, 1, 1, 64, sel[:, None], None if selg is None else selg[:, None], T)
    for t in range(T):
        codes, _ = O.block_table(lay, tm, L - 1, 1, 1, 64, sel[t][None], None if selg is None else selg[t][None])
        _compare(codes, table[t], cnt[t], lst[t])
