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
