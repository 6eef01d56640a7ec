"""GPU parity of selective unfolding at prefill scale: gsa_select_prefill
(MFMA scores at fp32 accuracy, per-row top-k) against the oracle's selection, and
gsa_attn_prefill_unfolded (unfolded raws attended first, then the MFMA prefill
of the fixed part starting from that partial) against the oracle's attention
with the GPU's selection; protocol and tolerances of gsa_testutil."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import LSE_TOL, TOL, assert_close, check_selection, to_dev

pytestmark = pytest.mark.gpu

SMALL = [
    # layout, L, B, Hq, Hkv, d
    (dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=3), 4 + 300 * 5 + 3, 1, 6, 2, 128),
    (dict(n_sink=16, chunk_len=8, gists=1, window=40, top_k=16), 16 + 200 * 9 + 5, 2, 4, 2, 128),
    (dict(n_sink=0, chunk_len=2, gists=1, window=3, top_k=16), 600 * 3 + 1, 1, 2, 1, 64),
    (dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=16), 128 + 400 * 5, 1, 3, 1, 128),
    (dict(n_sink=3, chunk_len=5, gists=1, window=7, top_k=28), 3 + 150 * 6 + 2, 1, 4, 2, 128),
    (dict(n_sink=2, chunk_len=3, gists=1, window=1, top_k=8), 2 + 500 * 4 + 1, 2, 8, 2, 64),
]


def _tables(layout, L, q_begin, q_len):
    fixed = dict(layout, top_k=0)
    bm, bn = gsa.prefill_tile(torch.bfloat16, 128)
    return gsa.build_layout(fixed, L, q_begin, q_len, bm, bn), (bm, bn)


def _run(layout, q, k, v, q_begin=0, out_dtype=torch.float32):
    B, Nq, Hq, d = q.shape
    L = k.shape[1]
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    scale = 1 / math.sqrt(d)
    sel = gsa.select_prefill(layout, tq, tk, L, q_begin, scale)
    tables, (bm, bn) = _tables(layout, L, q_begin, Nq)
    o, lse = gsa.attn_prefill_unfolded(layout, tq, tk, tv, sel, tables, bm, bn, q_begin, scale,
                                       out_dtype=out_dtype)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_unfolded_prefill_small_all_rows(case):
    layout, L, B, Hq, Hkv, d = SMALL[case]
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=200 + case, dtype="bf16")
    sel, o, lse = _run(layout, q, k, v)
    pos = list(range(L))
    scale = 1 / math.sqrt(d)
    check_selection(lay, tm, q, k, pos, scale, sel)
    ref, ref_lse = O.attend(lay, tm, q, k, v, pos, scale, sel)
    assert_close(o, ref, TOL["bf16"], what=f"unfolded prefill case {case}")
    assert_close(lse, ref_lse, LSE_TOL["bf16"], what=f"unfolded prefill lse case {case}")


def test_unfolded_prefill_query_offset_bf16_out():
    layout, L, B, Hq, Hkv, d = SMALL[1]
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=250, dtype="bf16")
    qb, ql = 333, 900
    sel, o, lse = _run(layout, q[:, qb:qb + ql], k, v, q_begin=qb, out_dtype=torch.bfloat16)
    pos = list(range(qb, qb + ql))
    scale = 1 / math.sqrt(d)
    check_selection(lay, tm, q[:, qb:qb + ql], k, pos, scale, sel)
    ref, _ = O.attend(lay, tm, q[:, qb:qb + ql], k, v, pos, scale, sel)
    assert_close(o, ref, TOL["bf16"], bf16_out=True, what="offset unfolded prefill")


def test_select_prefill_agrees_with_score_select():
    """Both selection paths on the same rows: identical except where both are
    valid near-top-k choices (gap < 1e-3)."""
    layout, L, B, Hq, Hkv, d = SMALL[3]
    q, k, _ = inputs.random_qkv(B, L, Hq, Hkv, d, seed=260, dtype="bf16")
    tq, tk = to_dev(q, "bf16"), to_dev(k, "bf16")
    a = gsa.select_prefill(layout, tq, tk, L, 0).cpu().numpy()
    b, _, _ = gsa.score_select(layout, tq, tk, L, 0)
    b = b.cpu().numpy()
    diff = (a != b).any(axis=-1)
    assert diff.mean() < 0.01
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    rows = sorted(set(np.nonzero(diff)[2].tolist()))[:50]
    if rows:
        check_selection(lay, tm, q[:, rows], k, rows, 1 / math.sqrt(d), a[:, :, rows])


def test_k16_workload_sampled_rows():
    """The 32K k=16 workload in the benchmarked configuration; the oracle
    checks every KV head's selection and every head's output on a sample of
    rows (first and last query tiles included)."""
    w = configs.LLAMA3B_K16_PREFILL
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q, k, v = inputs.prefill_inputs(w, seed=1)
    sel, o, lse = _run(w.layout, q, k, v, out_dtype=torch.bfloat16)
    rng = np.random.default_rng(1)
    rows = sorted(set([0, 1, 130, 131, 600, L // 2, L - 129, L - 2, L - 1]
                      + rng.choice(L, 16, replace=False).tolist()))
    scale = 1 / math.sqrt(w.d)
    check_selection(lay, tm, q[:, rows], k, rows, scale, sel[:, :, rows])
    ref, ref_lse = O.attend(lay, tm, q, k, v, list(range(L)), scale, sel, rows=rows)
    assert_close(o[:, rows], ref[:, rows], TOL["bf16"], bf16_out=True, what="k16 workload")
    assert_close(lse[:, :, rows], ref_lse[:, :, rows], LSE_TOL["bf16"], what="k16 workload lse")
    assert (sel >= -1).all() and (sel < 8192).all()


@pytest.mark.parametrize("layout", [dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=5),
                                    dict(n_sink=2, chunk_len=3, gists=1, window=8, top_k=20)])
def test_select_prefill_exact_ties_pick_lowest_chunks(layout):
    """Every gist key of a KV head equal: all candidates of a row tie, so the
    (score desc, chunk index asc) rule alone decides, and the kernel must keep
    each row's lowest chunk indices exactly as the oracle does."""
    B, Hq, Hkv, d = 1, 4, 2, 128
    lay = O.Layout.of(layout)
    L = layout["n_sink"] + 120 * (layout["chunk_len"] + 1) + 2
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(B, L, Hq, Hkv, d, seed=270, dtype="bf16")
    gpos = [g[0] for g in tm.chunk_gists if len(g)]
    k[:, gpos] = k[:, gpos[:1]]
    scale = 1 / math.sqrt(d)
    sel = gsa.select_prefill(layout, to_dev(q, "bf16"), to_dev(k, "bf16"), L, 0, scale).cpu().numpy()
    ref = O.select(lay, tm, q, k, list(range(L)), scale)["sel"]
    assert (sel == ref).all(), f"{int((sel != ref).any(axis=-1).sum())} rows differ"


def test_select_prefill_nan_gist_keys_rank_last():
    """A NaN gist key gives its chunk a NaN score, which ranks below every
    finite one (as -inf): each row keeps the top-k of its finite candidates,
    topped up with NaN ones (lowest ids first) where there are too few."""
    layout = dict(n_sink=2, chunk_len=4, gists=1, window=4, top_k=4)
    L = 2 + 40 * 5 + 1
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, _ = inputs.random_qkv(1, L, 4, 2, 128, seed=21, dtype="bf16")
    nan_chunks = {1, 3, 17}
    for m in nan_chunks:
        k[0, tm.chunk_gists[m][0], :, :] = np.nan
    scale = 1 / math.sqrt(128)
    sel = gsa.select_prefill(layout, to_dev(q, "bf16"), to_dev(k, "bf16"), L, 0, scale).cpu().numpy()
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
