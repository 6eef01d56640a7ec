"""GPU parity: gist scoring + per-KV-group top-k vs the oracle."""
import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import check_selection, dev, to_dev

pytestmark = pytest.mark.gpu


def _run(layout, q, k, L, q_begin, scale, dtype, cache=False, want_scores=False):
    tq, tk = to_dev(q, dtype), to_dev(k, dtype)
    sel, selg, sc = gsa.score_select(layout, tq, tk, L, q_begin, scale, cache_layout=cache,
                                     want_scores=want_scores)
    torch.cuda.synchronize()
    return (sel.cpu().numpy(), None if selg is None else selg.cpu().numpy(),
            None if sc is None else sc.cpu().numpy())


def test_tiny_prefill_every_row():
    w = configs.TINY_PREFILL_F32
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q, k, _ = inputs.prefill_inputs(w, seed=0)
    scale = 1 / np.sqrt(w.d)
    sel, _, sc = _run(w.layout, q, k, L, 0, scale, "f32", want_scores=True)
    check_selection(lay, tm, q, k, list(range(L)), scale, sel)
    # scores themselves: fp32 vs fp64 definition, candidates only
    for i in (40, 100, 300, 547):
        cands = O.chunk_candidates(lay, tm, i)
        ref = O.gist_scores(q[0, i, 0:1], k[0, :, 0], tm.chunk_gists, cands, scale)
        for m in cands:
            assert abs(sc[0, 0, i, m] - ref[m]) < 1e-5
        assert np.all(np.isneginf(sc[0, 0, i, len(cands):]))


@pytest.mark.parametrize("d,dtype,G,g", [(64, "bf16", 4, 1), (128, "bf16", 2, 1), (128, "f32", 1, 2),
                                         (64, "f32", 3, 3)])
def test_random_layouts(d, dtype, G, g):
    layout = dict(n_sink=3, chunk_len=5, gists=g, window=9, top_k=7)
    L = 3 + 150 * (5 + g) + 4
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    Hkv = 2
    q, k, _ = inputs.random_qkv(2, L, G * Hkv, Hkv, d, seed=d + G, dtype=dtype)
    rows = list(range(0, L, 7)) + [L - 1]
    qs = q[:, rows]
    # query rows are contiguous in the ABI: run all rows, compare a sample
    sel, _, _ = _run(layout, q, k, L, 0, 0.3, dtype)
    check_selection(lay, tm, qs, k, rows, 0.3, sel[:, :, rows])


def test_candidates_fewer_than_k_and_q_begin():
    layout = dict(n_sink=2, chunk_len=3, gists=1, window=2, top_k=5)
    L = 2 + 12 * 4
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 2, 1, 64, seed=1, dtype="bf16")
    qb = 4
    sel, _, _ = _run(layout, q[:, qb:], k, L, qb, 0.2, "bf16")
    check_selection(lay, tm, q[:, qb:], k, list(range(qb, L)), 0.2, sel)
    # chunk 0 is positions 2..5 (gist at 5): no candidate at 4 or 5, one at 6
    assert (sel[0, 0, 0] == -1).all() and (sel[0, 0, 1] == -1).all()
    assert sel[0, 0, 2][0] == 0 and (sel[0, 0, 2][1:] == -1).all()


def test_exact_ties_break_to_lowest_index():
    """Ternary q and k: scores are exact in any precision, so ties are real."""
    layout = dict(n_sink=1, chunk_len=2, gists=1, window=1, top_k=6)
    L = 1 + 200 * 3 + 1
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, _ = inputs.ternary_qkv(2, L, 4, 2, 64, seed=9)
    k = k * 0  # flatten: every gist key the same small-integer vector per head ...
    k[:, :, :, :3] = 1.0
    rng = np.random.default_rng(2)
    k[:, rng.choice(L, 150, replace=False), :, 3] = 1.0   # ... except some with a bigger score
    sel, _, _ = _run(layout, q[:, -1:], k, L, L - 1, 0.125, "bf16")
    ref = O.select(lay, tm, q[:, -1:], k, [L - 1], 0.125)
    assert np.array_equal(sel, ref["sel"])


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
def test_decode_workloads_full(w):
    """The full decode workloads: every (batch, KV head) group."""
    x = inputs.decode_inputs(w, seed=3 if not w.hierarchical else 4)
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    scale = 1 / np.sqrt(w.d)
    sel, selg, _ = _run(w.layout, x["q"], x["k"], L, L - 1, scale, w.dtype, cache=True)
    kk = x["k"].transpose(0, 2, 1, 3)
    n_acc = check_selection(lay, tm, x["q"][:, None], kk, [L - 1], scale, sel, selg)
    assert n_acc <= w.batch * w.hkv // 4
    hits = np.mean([len(set(sel[b, h, 0]) & set(x["plant_chunks"][b]))
                    for b in range(w.batch) for h in range(w.hkv)])
    assert hits > 4   # the planted chunks are found (statistical sanity)


def test_nan_gist_keys_rank_last():
    """A NaN gist key gives its chunk a NaN score, which ranks below every
    finite one (as -inf): the chosen ids stay distinct candidates, ascending,
    and equal the top-k of the finite candidates, topped up with the NaN ones
    (lowest ids first) where there are too few."""
    layout = dict(n_sink=2, chunk_len=4, gists=1, window=4, top_k=4)
    L = 2 + 40 * 5 + 1
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 4, 2, 128, seed=21, dtype="bf16")
    nan_chunks = {1, 3, 17}
    for m in nan_chunks:
        k[0, tm.chunk_gists[m][0], :, :] = np.nan
    scale = 1 / np.sqrt(128)
    sel, _, _ = _run(layout, q, k, L, 0, scale, "bf16")
    for h in range(2):
        for i in range(L):
            cands = O.chunk_candidates(lay, tm, i)
            finite = [m for m in cands if m not in nan_chunks]
            s = O.gist_scores(q[0, i, 2 * h:2 * h + 2], k[0, :, h], tm.chunk_gists, finite, scale)
            chosen, gap = O.top_k(s, 4)
            fill = sorted(m for m in cands if m in nan_chunks)[:4 - len(chosen)]
            want = sorted(chosen + fill) + [-1] * (4 - len(chosen) - len(fill))
            got = sel[0, h, i].tolist()
            if got != want:
                assert gap < 1e-3, f"row {i} head {h}: gpu {got} want {want} (gap {gap:.2e})"
                picked = [x for x in got if x >= 0]
                assert len(set(picked)) == len(picked) and set(picked) <= set(cands)


def test_two_level_exact_ties_break_to_lowest_ids():
    """Ternary inputs with a power-of-two scale make every score exact in fp32,
    so ties are real at both levels: kept groups and unfolded chunks must equal
    the oracle's exactly (lowest ids win), with no near-tie allowance."""
    layout = dict(n_sink=1, chunk_len=2, gists=1, window=3, top_k=5, l2_chunks=4, l2_gists=1,
                  l2_top_k=3)
    P2 = 4 * 3 + 1
    L = 1 + 40 * P2 + 2
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, _ = inputs.ternary_qkv(2, L, 4, 2, 64, seed=13)
    rows = list(range(L - 6, L))
    qb = rows[0]
    sel, selg, _ = _run(layout, q[:, qb:], k, L, qb, 0.125, "bf16")
    ref = O.select(lay, tm, q[:, qb:], k, rows, 0.125)
    assert np.array_equal(selg, ref["sel_groups"])
    assert np.array_equal(sel, ref["sel"])
    # all keys equal: every score ties, the lowest complete groups and their
    # lowest chunks win
    kk = np.ones_like(k)
    sel, selg, _ = _run(layout, q[:, qb:], kk, L, qb, 0.125, "bf16")
    assert (selg[:, :, :, :] == np.array([0, 1, 2])).all()
    assert (sel == np.array([0, 1, 2, 3, 4])).all()
