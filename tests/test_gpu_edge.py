"""GPU parity on degenerate and extreme inputs: a sequence shorter than the
sinks, no complete chunk, a window of 0 (the query sees only itself beyond
sinks and gists), a single position, fewer candidate chunks than top_k, no
sinks, the largest top_k (64, and 32 groups kept at level 2), and an empty
query range; decode of a one-position cache and of a cache still inside the
sinks.  Every row is checked against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import inputs
from gsa_testutil import LSE_TOL, TOL, assert_close, check_selection, dev, to_dev

pytestmark = pytest.mark.gpu

EDGE_PREFILL = [
    # layout, L, B, Hq, Hkv, d, dtype
    (dict(n_sink=64, chunk_len=4, gists=1, window=16, top_k=0), 40, 1, 4, 2, 128, "bf16"),
    (dict(n_sink=4, chunk_len=16, gists=1, window=8, top_k=2), 4 + 10, 1, 2, 1, 128, "bf16"),
    (dict(n_sink=2, chunk_len=4, gists=1, window=0, top_k=0), 2 + 30 * 5 + 2, 1, 2, 1, 128, "bf16"),
    (dict(n_sink=4, chunk_len=8, gists=1, window=16, top_k=0), 1, 1, 2, 1, 128, "bf16"),
    (dict(n_sink=2, chunk_len=8, gists=1, window=4, top_k=6), 2 + 3 * 9 + 4, 1, 2, 1, 64, "bf16"),
    (dict(n_sink=0, chunk_len=4, gists=1, window=1, top_k=2), 40 * 5 + 3, 1, 2, 1, 128, "bf16"),
    (dict(n_sink=64, chunk_len=4, gists=1, window=16, top_k=0), 40, 1, 2, 1, 64, "f32"),
    (dict(n_sink=3, chunk_len=4, gists=1, window=0, top_k=2, l2_chunks=2, l2_gists=1, l2_top_k=1),
     3 + 4 * 11 + 5, 1, 2, 1, 128, "bf16"),
    # the largest selections the library takes: top_k 64; two levels with 32 groups kept
    (dict(n_sink=4, chunk_len=4, gists=1, window=8, top_k=64), 4 + 200 * 5 + 3, 1, 4, 2, 128, "bf16"),
    (dict(n_sink=2, chunk_len=2, gists=1, window=4, top_k=64, l2_chunks=4, l2_gists=1, l2_top_k=32),
     2 + 80 * 13 + 5, 1, 2, 1, 128, "bf16"),
]


def _prefill(layout, q, k, v, dtype, scale):
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    bm, bn = gsa.prefill_tile(torch.bfloat16 if dtype == "bf16" else torch.float32, d)
    sel = selg = None
    n_tables = 1
    if int(layout.get("top_k", 0)) > 0 or int(layout.get("l2_chunks", 0)) > 0:
        sel, selg, _ = gsa.score_select(layout, tq, tk, L, 0, scale)
        n_tables = B * Hkv
    tables = gsa.build_layout(layout, L, 0, Nq, bm, bn, sel, selg, n_tables)
    o, lse = gsa.attn_prefill(layout, tq, tk, tv, tables, bm, bn, sel, selg, 0, scale)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), lse.cpu().numpy(), None if sel is None else sel.cpu().numpy(),
            None if selg is None else selg.cpu().numpy())


@pytest.mark.parametrize("case", range(len(EDGE_PREFILL)))
def test_prefill_degenerate_layouts_all_rows(case):
    layout, L, B, Hq, Hkv, d, dtype = EDGE_PREFILL[case]
    print(f"edge prefill case {case}: {layout} L={L} d={d} {dtype}", flush=True)
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=900 + case, dtype=dtype)
    scale = 1 / math.sqrt(d)
    o, lse, sel, selg = _prefill(layout, q, k, v, dtype, scale)
    pos = list(range(L))
    if sel is not None:
        check_selection(lay, tm, q, k, pos, scale, sel, selg)
    ref, ref_lse = O.attend(lay, tm, q, k, v, pos, scale, sel, selg)
    assert_close(o, ref, TOL[dtype], what=f"edge prefill case {case}")
    assert_close(lse, ref_lse, LSE_TOL[dtype], what=f"edge lse case {case}")
    assert np.array_equal(o[:, 0], v[:, 0].repeat(Hq // Hkv, axis=1))   # position 0 sees only itself


def test_prefill_empty_query_range():
    """q_len = 0 through the binding (zero-size tensors): every call succeeds
    and launches nothing."""
    layout = dict(n_sink=4, chunk_len=4, gists=1, window=8, top_k=2)
    L, B, Hq, Hkv, d = 4 + 20 * 5, 1, 2, 1, 128
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=7, dtype="bf16")
    tq, tk, tv = to_dev(q[:, :0], "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    sel, selg, _ = gsa.score_select(layout, tq, tk, L, 5, 0.1)
    tables = gsa.build_layout(layout, L, 5, 0, 128, 64, sel, None, B * Hkv)
    o, lse = gsa.attn_prefill(layout, tq, tk, tv, tables, 128, 64, sel, None, 5, 0.1)
    torch.cuda.synchronize()
    assert sel.numel() == 0 and o.numel() == 0 and lse.numel() == 0


EDGE_DECODE = [
    # layout, kv_len, B, Hq, Hkv, d
    (dict(n_sink=4, chunk_len=8, gists=1, window=16, top_k=3), 1, 2, 4, 2, 128),
    (dict(n_sink=64, chunk_len=8, gists=1, window=16, top_k=3), 40, 1, 4, 1, 128),
    (dict(n_sink=4, chunk_len=16, gists=1, window=8, top_k=2), 4 + 16, 1, 2, 1, 64),
    (dict(n_sink=2, chunk_len=4, gists=1, window=0, top_k=5), 2 + 30 * 5 + 2, 2, 4, 2, 128),
]


@pytest.mark.parametrize("case", range(len(EDGE_DECODE)))
def test_decode_degenerate_caches(case):
    """Split-K decode (after gsa_score_select) and the fused step on the same
    degenerate caches, both against the oracle."""
    layout, L, B, Hq, Hkv, d = EDGE_DECODE[case]
    print(f"edge decode case {case}: {layout} kv_len={L} d={d}", flush=True)
    q = inputs.random_qkv(B, 1, Hq, Hkv, d, seed=60 + case, dtype="bf16")[0][:, 0]
    kc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=70 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    vc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=80 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    scale = 1 / math.sqrt(d)
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    kk, vv = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
    sel, selg, _ = gsa.score_select(layout, tq, tk, L, L - 1, scale, cache_layout=True)
    o, lse = gsa.attn_decode(layout, tq, tk, tv, sel, selg, scale)
    o2, lse2, sel2, _ = gsa.decode_step(layout, tq, tk, tv, scale)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    check_selection(lay, tm, q[:, None], kk, [L - 1], scale, sel_np, None)
    assert np.array_equal(sel2.cpu().numpy().reshape(sel_np.shape), sel_np)
    ref, ref_lse = O.attend(lay, tm, q[:, None], kk, vv, [L - 1], scale, sel_np, None)
    for out, out_lse, name in ((o, lse, "decode"), (o2, lse2, "decode step")):
        assert_close(out.cpu().numpy(), ref[:, 0], TOL["bf16"], what=f"edge {name} case {case}")
        assert_close(out_lse.cpu().numpy(), ref_lse[:, :, 0], LSE_TOL["bf16"], what=f"edge {name} lse case {case}")
