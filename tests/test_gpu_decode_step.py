"""GPU parity of the fused decode step (gsa_decode_step: selection at one or
two levels plus split-K attention, every visible row read once) against the
fp64 oracle, with the comparison protocol of gsa_testutil."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import LSE_TOL, TOL, assert_close, check_selection, dev, to_dev

pytestmark = pytest.mark.gpu


def _check(layout, q, kc, vc, L, scale, out_dtype=torch.float32):
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
    o, lse, sel, selg = gsa.decode_step(layout, tq, tk, tv, scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o, lse, sel = o.float().cpu().numpy(), lse.cpu().numpy(), sel.cpu().numpy()
    selg = None if selg is None else selg.cpu().numpy()
    kk, vv = kc.transpose(0, 2, 1, 3), vc.transpose(0, 2, 1, 3)
    n_acc = check_selection(lay, tm, q[:, None], kk, [L - 1], scale, sel, selg)
    ref, ref_lse = O.attend(lay, tm, q[:, None], kk, vv, [L - 1], scale, sel, selg)
    assert_close(o, ref[:, 0], TOL["bf16"], bf16_out=out_dtype == torch.bfloat16, what="decode step")
    assert_close(lse, ref_lse[:, :, 0], LSE_TOL["bf16"], what="decode step lse")
    return sel, selg, n_acc


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_decode_step_workloads_full(w, out_dtype):
    x = inputs.decode_inputs(w, seed=11)
    sel, selg, n_acc = _check(w.layout, x["q"], x["k"], x["v"], w.seq_len, 1 / math.sqrt(w.d),
                              torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    assert n_acc <= w.batch * w.hkv // 4
    hits = np.mean([len(set(sel[b, h, 0]) & set(x["plant_chunks"][b]))
                    for b in range(w.batch) for h in range(w.hkv)])
    assert hits > 4   # the planted chunks are found (statistical sanity)


STEP = [
    # layout, L, B, Hq, Hkv, d
    (dict(n_sink=4, chunk_len=8, gists=1, window=16, top_k=5), 4 + 70 * 9 + 1, 3, 8, 2, 128),
    (dict(n_sink=0, chunk_len=3, gists=2, window=1, top_k=3), 40 * 5 + 3, 2, 4, 4, 64),
    (dict(n_sink=6, chunk_len=16, gists=1, window=300, top_k=2), 6 + 20 * 17 + 1, 1, 16, 1, 128),
    (dict(n_sink=2, chunk_len=4, gists=1, window=8, top_k=6, l2_chunks=3, l2_gists=2, l2_top_k=3),
     2 + 25 * 17 + 1, 2, 6, 2, 128),
    (dict(n_sink=2, chunk_len=4, gists=3, window=9, top_k=4), 2 + 400 * 7 + 2, 2, 8, 2, 128),
    (dict(n_sink=1, chunk_len=2, gists=1, window=5, top_k=64), 1 + 3000 * 3 + 1, 1, 4, 1, 64),
    (dict(n_sink=3, chunk_len=5, gists=2, window=40, top_k=7, l2_chunks=4, l2_gists=3, l2_top_k=5),
     3 + 60 * 31 + 4, 2, 4, 2, 64),
    (dict(n_sink=8, chunk_len=4, gists=1, window=4, top_k=3), 8 + 2 * 5 + 1, 2, 4, 2, 128),
]


@pytest.mark.parametrize("case", range(len(STEP)))
def test_decode_step_small_layouts(case):
    """Ragged layouts: several gists per chunk (candidates that straddle
    blocks), level-2 gists per group, a window wider than the sequence,
    k = 64 over thousands of candidates, fewer candidates than k."""
    layout, L, B, Hq, Hkv, d = STEP[case]
    q = inputs.random_qkv(B, 1, Hq, Hkv, d, seed=60 + case, dtype="bf16")[0][:, 0]
    kc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=70 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    vc = inputs.random_qkv(B, L, Hkv, Hkv, d, seed=80 + case, dtype="bf16")[1].transpose(0, 2, 1, 3).copy()
    _check(layout, q, kc, vc, L, 1 / math.sqrt(d))


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
def test_decode_step_matches_separate_calls(w):
    """The fused step against gsa_score_select + gsa_attn_decode on the same
    inputs: selections agree except at near-ties (where both are validated
    near-top-k), outputs agree to the bf16 bar wherever the selections do."""
    x = inputs.decode_inputs(w, seed=12)
    L = w.seq_len
    tq, tk, tv = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    scale = 1 / math.sqrt(w.d)
    o1, _, s1, g1 = gsa.decode_step(w.layout, tq, tk, tv, scale)
    s2, g2, _ = gsa.score_select(w.layout, tq, tk, L, L - 1, scale, cache_layout=True)
    o2, _ = gsa.attn_decode(w.layout, tq, tk, tv, s2, g2, scale)
    torch.cuda.synchronize()
    same = (s1 == s2).all(dim=-1)
    if g1 is not None:
        same &= (g1 == g2).all(dim=-1)
    same = same[:, :, 0].cpu().numpy()
    assert same.mean() >= 0.9
    d1, d2 = o1.cpu().numpy(), o2.cpu().numpy()
    G = w.hq // w.hkv
    for b in range(w.batch):
        for h in range(w.hkv):
            if same[b, h]:
                assert np.abs(d1[b, h * G:(h + 1) * G] - d2[b, h * G:(h + 1) * G]).max() <= 1e-2


@pytest.mark.parametrize("w", [configs.SELECTIVE_DECODE, configs.HIER_DECODE], ids=lambda w: w.name)
def test_decode_step_workspace_reuse_and_graph_replay(w):
    """Counters come back to zero after every call: repeated eager calls and
    replays of a captured graph give bit-identical outputs and selections."""
    x = inputs.decode_inputs(w, seed=5)
    L = w.seq_len
    tq, tk, tv = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    scale = 1 / math.sqrt(w.d)
    need = gsa.decode_step_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    o, lse, sel, selg = gsa.decode_step(w.layout, tq, tk, tv, scale, workspace=ws)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, sel) + ((selg,) if selg is not None else ())]
    n_counters = 2 * w.batch * w.hkv
    outs = (o, lse, sel, selg)
    for _ in range(3):
        o.zero_()
        sel.zero_()
        gsa.decode_step(w.layout, tq, tk, tv, scale, workspace=ws, out=outs)
        torch.cuda.synchronize()
        for a, b in zip(ref, (o, lse, sel, selg)):
            assert torch.equal(a, b)
        assert int(ws[:4 * n_counters].view(torch.int32).abs().sum()) == 0, "counters not reset"
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            gsa.decode_step(w.layout, tq, tk, tv, scale, workspace=ws, out=outs)
    torch.cuda.current_stream().wait_stream(st)
    for _ in range(3):
        o.zero_()
        sel.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (o, lse, sel, selg)):
            assert torch.equal(a, b)
        assert int(ws[:4 * n_counters].view(torch.int32).abs().sum()) == 0, "counters not reset"
