"""GPU parity: block-sparse prefill and split-K decode vs the fp64 oracle.

The oracle is evaluated with the GPU's own (validated) selection; see
gsa_testutil for the protocol and tolerances."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import LSE_TOL, TOL, assert_close, check_selection, dev, to_dev

pytestmark = pytest.mark.gpu


def _prefill(layout, q, k, v, dtype, scale, out_dtype=torch.float32, q_begin=0, tile=None):
    """Full GPU path: selection (if any), table, attention.  Returns numpy."""
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bm, bn = tile or gsa.prefill_tile(tdt, d)
    sel = selg = None
    n_tables = 1
    if int(layout.get("top_k", 0)) > 0 or int(layout.get("l2_chunks", 0)) > 0:
        sel, selg, _ = gsa.score_select(layout, tq, tk, L, q_begin, scale)
        n_tables = B * Hkv
    tables = gsa.build_layout(layout, L, q_begin, Nq, bm, bn, sel, selg, n_tables)
    o, lse = gsa.attn_prefill(layout, tq, tk, tv, tables, bm, bn, sel, selg, q_begin, scale,
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), lse.cpu().numpy(),
            None if sel is None else sel.cpu().numpy(), None if selg is None else selg.cpu().numpy())


def test_tiny_prefill_f32_all_rows():
    """The tiny fp32 workload end to end, every row, 1e-4."""
    w = configs.TINY_PREFILL_F32
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q, k, v = inputs.prefill_inputs(w, seed=0)
    scale = 1 / math.sqrt(w.d)
    o, lse, sel, _ = _prefill(w.layout, q, k, v, "f32", scale)
    pos = list(range(L))
    check_selection(lay, tm, q, k, pos, scale, sel)
    ref, ref_lse = O.attend(lay, tm, q, k, v, pos, scale, sel)
    assert_close(o, ref, TOL["f32"], what="tiny fp32 prefill")
    assert_close(lse, ref_lse, LSE_TOL["f32"], what="tiny fp32 lse")
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])   # row 0 sees only itself


SMALL = [
    # layout, L, B, Hq, Hkv, d, dtype, q_scale
    (dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0), 128 + 500 * 5 + 0, 1, 6, 2, 128, "bf16", 1.0),
    (dict(n_sink=16, chunk_len=8, gists=1, window=64, top_k=0), 16 + 300 * 9 + 7, 2, 4, 1, 128, "bf16", 4.0),
    (dict(n_sink=4, chunk_len=5, gists=2, window=20, top_k=0), 4 + 210 * 7 + 3, 1, 4, 2, 64, "bf16", 1.0),
    (dict(n_sink=8, chunk_len=16, gists=1, window=32, top_k=4), 8 + 90 * 17 + 9, 1, 4, 2, 128, "bf16", 1.0),
    (dict(n_sink=3, chunk_len=4, gists=1, window=10, top_k=3, l2_chunks=4, l2_gists=1, l2_top_k=2),
     3 + 30 * 21 + 6, 1, 2, 1, 128, "bf16", 1.0),
    (dict(n_sink=2, chunk_len=6, gists=1, window=12, top_k=2), 2 + 60 * 7 + 1, 1, 3, 1, 64, "f32", 1.0),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_prefill_small_layouts_all_rows(case, out_dtype):
    """Several tiles and a ragged tail, every row checked."""
    layout, L, B, Hq, Hkv, d, dtype, qs = SMALL[case]
    if out_dtype == "bf16" and dtype == "f32":
        pytest.skip("bf16 output is for bf16 inputs")
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=100 + case, dtype=dtype, q_scale=qs)
    if dtype == "bf16":
        q = inputs.round_bf16(q)
    scale = 1 / math.sqrt(d)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    o, lse, sel, selg = _prefill(layout, q, k, v, dtype, scale, out_dtype=odt)
    pos = list(range(L))
    if sel is not None:
        check_selection(lay, tm, q, k, pos, scale, sel, selg)
    ref, ref_lse = O.attend(lay, tm, q, k, v, pos, scale, sel, selg)
    assert_close(o, ref, TOL[dtype], bf16_out=out_dtype == "bf16", what=f"prefill case {case}")
    assert_close(lse, ref_lse, LSE_TOL[dtype], what=f"lse case {case}")


def test_prefill_query_offset():
    """Query rows [q_begin, q_begin + q_len) of a longer sequence."""
    layout = dict(n_sink=32, chunk_len=4, gists=1, window=48, top_k=0)
    L = 32 + 400 * 5
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(1, L, 4, 2, 128, seed=7, dtype="bf16")
    qb, ql = 777, 700
    o, lse, _, _ = _prefill(layout, q[:, qb:qb + ql], k, v, "bf16", 0.09, q_begin=qb)
    ref, _ = O.attend(lay, tm, q[:, qb:qb + ql], k, v, list(range(qb, qb + ql)), 0.09)
    assert_close(o, ref, TOL["bf16"], what="offset prefill")


@pytest.mark.parametrize("w", [configs.LLAMA3B_K0_PREFILL, configs.LLAMA8B_K0_PREFILL],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_prefill_full_size_sampled_rows(w, out_dtype):
    """The 32K workloads in the benchmarked launch configuration; the oracle
    checks every head of a sample of rows (first and last tiles included)."""
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    tm = O.type_map(lay, L)
    q, k, v = inputs.prefill_inputs(w, seed=1)
    scale = 1 / math.sqrt(w.d)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    o, lse, _, _ = _prefill(w.layout, q, k, v, w.dtype, scale, out_dtype=odt)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 5, 127, 128, 129, 130, L // 2, L - 129, L - 128, L - 2, L - 1]
                      + rng.choice(L, 24, replace=False).tolist()))
    ref, ref_lse = O.attend(lay, tm, q, k, v, list(range(L)), scale, rows=rows)
    assert_close(o[:, rows], ref[:, rows], TOL["bf16"], bf16_out=out_dtype == "bf16",
                 what=f"{w.name} sampled rows")
    assert_close(lse[:, :, rows], ref_lse[:, :, rows], LSE_TOL["bf16"], what=f"{w.name} lse")
    assert np.isfinite(o).all()


# ---------------------------------------------------------------- decode
def _decode(layout, q, kc, vc, L, scale, out_dtype=torch.float32):
    tq, tk, tv = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
    sel, selg, _ = gsa.score_select(layout, tq, tk, L, L - 1, scale, cache_layout=True)
    o, lse = gsa.attn_decode(layout, tq, tk, tv, sel, selg, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy(),
            None if selg is None else selg.cpu().numpy())


def _check_decode(layout, q, kc, vc, L, scale, out_dtype=torch.float32):
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    o, lse, sel, selg = _decode(layout, q, kc, vc, L, scale, out_dtype)
    kk, vv = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3)
    check_selection(lay, tm, q[:, None], kk, [L - 1], scale, sel, selg)
    ref, ref_lse = O.attend(lay, tm, q[:, None], kk, vv, [L - 1], scale, sel, selg)
    assert_close(o, ref[:, 0], TOL["bf16"], bf16_out=out_dtype == torch.bfloat16, what="decode")
    assert_close(lse, ref_lse[:, :, 0], LSE_TOL["bf16"], what="decode lse")


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_decode_workloads_full(w, out_dtype):
    x = inputs.decode_inputs(w, seed=11)
    _check_decode(w.layout, x["q"], x["k"], x["v"], w.seq_len, 1 / math.sqrt(w.d),
                  torch.bfloat16 if out_dtype == "bf16" else torch.float32)


DEC = [
    (dict(n_sink=4, chunk_len=8, gists=1, window=16, top_k=5), 4 + 70 * 9 + 1, 3, 8, 2, 128),
    (dict(n_sink=0, chunk_len=3, gists=2, window=1, top_k=3), 40 * 5 + 3, 2, 4, 4, 64),
    (dict(n_sink=6, chunk_len=16, gists=1, window=300, top_k=2), 6 + 20 * 17 + 1, 1, 16, 1, 128),
    (dict(n_sink=2, chunk_len=4, gists=1, window=8, top_k=6, l2_chunks=3, l2_gists=2, l2_top_k=3),
     2 + 25 * 17 + 1, 2, 6, 2, 128),
    (dict(n_sink=2, chunk_len=4, gists=1, window=8, top_k=0), 2 + 90 * 5 + 3, 2, 4, 2, 128),
]


@pytest.mark.parametrize("case", range(len(DEC)))
def test_decode_small_layouts(case):
    layout, L, B, Hq, Hkv, d = DEC[case]
    rng_q = inputs.random_qkv(B, 1, Hq, Hkv, d, seed=30 + case, dtype="bf16")[0][:, 0]
    kc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=40 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    vc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=50 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    if int(layout["top_k"]) == 0:
        lay = O.Layout.of(layout)
        tm = O.type_map(lay, L)
        tq, tk, tv = to_dev(rng_q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
        o, _ = gsa.attn_decode(layout, tq, tk, tv, None, None, 1 / math.sqrt(d))
        torch.cuda.synchronize()
        ref, _ = O.attend(lay, tm, rng_q[:, None], kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3),
                          [L - 1], 1 / math.sqrt(d))
        assert_close(o.cpu().numpy(), ref[:, 0], TOL["bf16"], what="fixed-layout decode")
        return
    _check_decode(layout, rng_q, kc, vc, L, 1 / math.sqrt(d))


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
def test_decode_workspace_reuse_and_graph_replay(w):
    """One workspace across many calls: the completion counters must come back
    to zero after every call, so repeated calls (eager, then replays of a
    captured graph with eager work between them) give bit-identical outputs."""
    x = inputs.decode_inputs(w, seed=5)
    L = w.seq_len
    tq, tk, tv = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    scale = 1 / math.sqrt(w.d)
    sel, selg, _ = gsa.score_select(w.layout, tq, tk, L, L - 1, scale, cache_layout=True)
    need = gsa.decode_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    o = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=dev())
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev())
    gsa.attn_decode(w.layout, tq, tk, tv, sel, selg, scale, workspace=ws, out=(o, lse))
    torch.cuda.synchronize()
    ref_o, ref_lse = o.clone(), lse.clone()
    n_counters = w.batch * w.hkv
    for _ in range(3):
        o.zero_()
        gsa.attn_decode(w.layout, tq, tk, tv, sel, selg, scale, workspace=ws, out=(o, lse))
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
        assert int(ws[:4 * n_counters].view(torch.int32).abs().sum()) == 0, "counters not reset"
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            gsa.attn_decode(w.layout, tq, tk, tv, sel, selg, scale, workspace=ws, out=(o, lse))
    torch.cuda.current_stream().wait_stream(st)
    for _ in range(3):
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
        assert int(ws[:4 * n_counters].view(torch.int32).abs().sum()) == 0, "counters not reset"
