"""GPU parity of the prefill backward (dq, dk, dv) against the fp64 oracle
(oracle/gsa_backward.py; the block-mask variant against autograd-free fp64
formulas over the gzip oracle's mask): fixed layouts, layouts with top-k
unfolding at one and two levels, and block masks.

Inputs are bf16-exact (workloads.inputs), so the oracle sees the same numbers.
Tolerance (from the arithmetic): the kernels round P and dS to bf16 (relative
2^-9 per term) before the dV, dK and dQ products and take D from the
forward's output; sums are fp32.  Each gradient element is a sum of such
terms, so its error is bounded by about 2^-8 of the sum of the terms'
magnitudes.  The test takes that bound per tensor as GRAD_TOL = 1e-2 of the
largest reference magnitude (elementwise) and 4e-3 of the reference norm
(normwise).
"""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_backward as GB
from oracle import gsa_oracle as O
from oracle import gzip_mask as gm
from workloads import configs, inputs

from gsa_testutil import dev

pytestmark = pytest.mark.gpu

GRAD_TOL = {"max": 1e-2, "norm": 4e-3}


def assert_grad_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN"
    err = np.abs(got - ref)
    scale_max = max(np.abs(ref).max(), 1e-30)
    rel_norm = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    print(f"{what}: max err {err.max():.3e} ({err.max() / scale_max:.2e} of max), norm {rel_norm:.2e}")
    assert err.max() <= GRAD_TOL["max"] * scale_max, f"{what}: max err {err.max():.3e} vs max |ref| {scale_max:.3e}"
    assert rel_norm <= GRAD_TOL["norm"], f"{what}: normwise {rel_norm:.2e}"


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev()).to(torch.bfloat16)


def _forward_backward(layout, q, k, v, do, q_begin, o_dtype, grad_dtype):
    B, Nq, Hq, d = q.shape
    L = k.shape[1]
    tq, tk, tv, tdo = _bf(q), _bf(k), _bf(v), _bf(do)
    bm, bn = gsa.prefill_tile(torch.bfloat16, d)
    tables = gsa.build_layout(layout, L, q_begin, Nq, bm, bn, device=dev())
    o, lse = gsa.attn_prefill(layout, tq, tk, tv, tables, bm, bn, q_begin=q_begin, out_dtype=o_dtype)
    dq, dk, dv = gsa.attn_prefill_backward(layout, tq, tk, tv, o, tdo, lse, tables, bm, bn, q_begin=q_begin,
                                           grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return (t.float().cpu().numpy() for t in (dq, dk, dv))


SMALL = [
    # layout, L, B, Hq, Hkv, d, q_begin
    (dict(n_sink=4, chunk_len=4, gists=1, window=64, top_k=0), 4 + 150 * 5 + 3, 2, 4, 2, 128, 0),
    (dict(n_sink=2, chunk_len=8, gists=2, window=40, top_k=0), 2 + 60 * 10 + 7, 1, 3, 1, 64, 0),
    (dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0), 128 + 100 * 5, 1, 2, 2, 128, 0),
    (dict(n_sink=1, chunk_len=3, gists=1, window=5, top_k=0), 1 + 170 * 4 + 2, 1, 4, 4, 64, 130),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("o_dtype,grad_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                                (torch.float32, torch.bfloat16)])
def test_backward_small_layouts_all_rows(case, o_dtype, grad_dtype):
    layout, L, B, Hq, Hkv, d, q_begin = SMALL[case]
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=300 + case, dtype="bf16")
    do = inputs.round_bf16(np.random.default_rng(400 + case).standard_normal((B, L, Hq, d), dtype=np.float32))
    q, do = q[:, q_begin:], do[:, q_begin:]
    dq, dk, dv = _forward_backward(layout, q, k, v, do, q_begin, o_dtype, grad_dtype)
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    rq, rk, rv, _, _ = GB.attend_backward(lay, tm, q, k, v, do, list(range(q_begin, L)), 1 / math.sqrt(d))
    tag = f"case {case} o {o_dtype} g {grad_dtype}"
    assert_grad_close(dq, rq, "dq " + tag)
    assert_grad_close(dk, rk, "dk " + tag)
    assert_grad_close(dv, rv, "dv " + tag)


def test_blockmask_backward_all_rows():
    B, L, Hq, Hkv, d, block, w = 2, 640, 4, 2, 64, 128, 1
    x = inputs.mixed_bytes(B, L, block, 55)
    _, flags = gsa.gzip_block_flags(x, block)
    masks = [gm.token_mask(gm.block_mask(flags[b].astype(bool), w), L, block) for b in range(B)]
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=56, dtype="bf16")
    do = inputs.round_bf16(np.random.default_rng(57).standard_normal((B, L, Hq, d), dtype=np.float32))
    tq, tk, tv, tdo = _bf(q), _bf(k), _bf(v), _bf(do)
    tables = gsa.build_block_mask(torch.from_numpy(flags).to(dev()), block, w, L, 0, L, 128, 64)
    o, lse = gsa.attn_prefill_blockmask(tq, tk, tv, tables, 128, 64)
    dq, dk, dv = gsa.attn_prefill_backward("blockmask", tq, tk, tv, o, tdo, lse, tables, 128, 64)
    torch.cuda.synchronize()
    # fp64 reference from the same derivative, over the gzip oracle's masks
    scale = 1 / math.sqrt(d)
    G = Hq // Hkv
    rq = np.zeros((B, L, Hq, d))
    rk = np.zeros((B, L, Hkv, d))
    rv = np.zeros((B, L, Hkv, d))
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            for i in range(L):
                idx = np.nonzero(masks[b][i])[0]
                kk, vv = k[b, idx, h].astype(np.float64), v[b, idx, h].astype(np.float64)
                qr, dr = q[b, i, hq].astype(np.float64), do[b, i, hq].astype(np.float64)
                s = kk @ qr * scale
                p = np.exp(s - s.max())
                p /= p.sum()
                dp = vv @ dr
                ds = p * (dp - dr @ (p @ vv))
                rq[b, i, hq] = scale * ds @ kk
                rk[b, idx, h] += scale * np.outer(ds, qr)
                rv[b, idx, h] += np.outer(p, dr)
    assert_grad_close(dq.cpu().numpy(), rq, "dq blockmask")
    assert_grad_close(dk.cpu().numpy(), rk, "dk blockmask")
    assert_grad_close(dv.cpu().numpy(), rv, "dv blockmask")


def test_backward_selection_layout_needs_sel():
    layout = dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=2)
    t = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device=dev())
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=dev())
    tables = (torch.zeros(1, dtype=torch.int8, device=dev()), torch.zeros(1, dtype=torch.int32, device=dev()),
              torch.zeros(1, dtype=torch.int32, device=dev()))
    with pytest.raises(gsa.GsaError) as e:
        gsa.attn_prefill_backward(layout, t, t, t, t, t, lse, tables, 128, 64)
    assert e.value.status == gsa.GSA_EINVAL


SEL = [
    # layout, L, B, Hq, Hkv, d, q_begin: selections from gsa_score_select, one table per (batch, KV head)
    (dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=3), 4 + 120 * 5 + 3, 2, 4, 2, 128, 0),
    (dict(n_sink=2, chunk_len=8, gists=2, window=20, top_k=4), 2 + 50 * 10 + 5, 1, 3, 1, 64, 37),
    (dict(n_sink=1, chunk_len=2, gists=1, window=3, top_k=5, l2_chunks=4, l2_gists=1, l2_top_k=3),
     1 + 40 * 13 + 6, 1, 4, 2, 128, 0),
]


@pytest.mark.parametrize("case", range(len(SEL)))
def test_backward_selection_layouts_all_rows(case):
    """Layouts with top-k unfolding (one and two levels): the forward with the
    GPU's selections and its tables, then the backward with the same, against
    the fp64 backward oracle over the same selections, every row."""
    layout, L, B, Hq, Hkv, d, q_begin = SEL[case]
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=500 + case, dtype="bf16")
    do = inputs.round_bf16(np.random.default_rng(600 + case).standard_normal((B, L, Hq, d), dtype=np.float32))
    q, do = q[:, q_begin:], do[:, q_begin:]
    Nq = L - q_begin
    scale = 1 / math.sqrt(d)
    tq, tk, tv, tdo = _bf(q), _bf(k), _bf(v), _bf(do)
    sel, selg, _ = gsa.score_select(layout, tq, tk, L, q_begin, scale)
    bm, bn = gsa.prefill_tile(torch.bfloat16, d)
    tables = gsa.build_layout(layout, L, q_begin, Nq, bm, bn, sel, selg, B * Hkv, device=dev())
    o, lse = gsa.attn_prefill(layout, tq, tk, tv, tables, bm, bn, sel, selg, q_begin, scale,
                              out_dtype=torch.float32)
    dq, dk, dv = gsa.attn_prefill_backward(layout, tq, tk, tv, o, tdo, lse, tables, bm, bn, q_begin=q_begin,
                                           scale=scale, grad_dtype=torch.float32, sel=sel, sel_groups=selg)
    torch.cuda.synchronize()
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    s_np = sel.cpu().numpy()
    g_np = None if selg is None else selg.cpu().numpy()
    rq, rk, rv, _, _ = GB.attend_backward(lay, tm, q, k, v, do, list(range(q_begin, L)), scale, s_np, g_np)
    tag = f"selection case {case}"
    assert_grad_close(dq.cpu().numpy(), rq, "dq " + tag)
    assert_grad_close(dk.cpu().numpy(), rk, "dk " + tag)
    assert_grad_close(dv.cpu().numpy(), rv, "dv " + tag)


def test_backward_workload_sampled():
    """The 3B-shape 32K fixed layout: dq of sampled rows (each needs only its
    row), and dk/dv of sampled raw keys well past the sinks (visible only to
    the queries of their window, all of which the oracle then evaluates)."""
    w = configs.LLAMA3B_K0_PREFILL
    L = w.seq_len
    q, k, v = inputs.prefill_inputs(w, seed=11)
    do = inputs.round_bf16(np.random.default_rng(12).standard_normal((w.batch, L, w.hq, w.d), dtype=np.float32))
    dq, dk, dv = _forward_backward(w.layout, q, k, v, do, 0, torch.bfloat16, torch.float32)
    lay = O.Layout.of(w.layout)
    tm = O.type_map(lay, L)
    scale = 1 / math.sqrt(w.d)
    rng = np.random.default_rng(13)
    rows = sorted(set(rng.integers(0, L, 6).tolist()) | {L - 1})
    rq, _, _, _, _ = GB.attend_backward(lay, tm, q[:, rows], k, v, do[:, rows], rows, scale)
    assert_grad_close(dq[:, rows], rq, "dq workload rows")
    typ = np.asarray(tm.typ)
    raws = np.nonzero(typ == O.RAW)[0]
    keys = [int(p) for p in rng.choice(raws[raws > 20000], 2, replace=False)]
    for p in keys:
        wrows = list(range(p, min(L, p + w.window)))
        _, rk, rv, _, _ = GB.attend_backward(lay, tm, q[:, wrows], k, v, do[:, wrows], wrows, scale)
        assert_grad_close(dk[:, p], rk[:, p], f"dk raw key {p}")
        assert_grad_close(dv[:, p], rv[:, p], f"dv raw key {p}")


UNF = [
    # layout, L, B, Hq, Hkv, d, q_begin: the unfolded forward and its backward
    (dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=3), 4 + 200 * 5 + 3, 2, 6, 2, 128, 0),
    (dict(n_sink=16, chunk_len=8, gists=1, window=40, top_k=16), 16 + 120 * 9 + 5, 1, 4, 2, 128, 0),
    (dict(n_sink=2, chunk_len=3, gists=2, window=7, top_k=8), 2 + 150 * 5 + 1, 1, 8, 2, 64, 101),
    (dict(n_sink=8, chunk_len=16, gists=1, window=24, top_k=4), 8 + 40 * 17 + 9, 1, 4, 1, 64, 0),
    (dict(n_sink=3, chunk_len=2, gists=1, window=12, top_k=6), 3 + 300 * 3 + 2, 1, 3, 1, 128, 0),
]


def _unfolded_forward_backward(layout, q, k, v, do, q_begin, grad_dtype):
    B, Nq, Hq, d = q.shape
    L = k.shape[1]
    scale = 1 / math.sqrt(d)
    tq, tk, tv, tdo = _bf(q), _bf(k), _bf(v), _bf(do)
    if layout["gists"] == 1:
        sel = gsa.select_prefill(layout, tq, tk, L, q_begin, scale)
    else:   # the prefill-scale selection takes one gist per chunk
        sel = gsa.score_select(layout, tq, tk, L, q_begin, scale)[0]
    bm, bn = gsa.prefill_tile(torch.bfloat16, d)
    fixed = gsa.build_layout(dict(layout, top_k=0), L, q_begin, Nq, bm, bn, device=dev())
    o, lse = gsa.attn_prefill_unfolded(layout, tq, tk, tv, sel, fixed, bm, bn, q_begin, scale,
                                       out_dtype=torch.float32)
    dq, dk, dv = gsa.attn_prefill_unfolded_backward(layout, tq, tk, tv, o, tdo, lse, sel, fixed, bm, bn, q_begin,
                                                    scale, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()


@pytest.mark.parametrize("case", range(len(UNF)))
@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_unfolded_backward_small_all_rows(case, grad_dtype):
    """gsa_attn_prefill_unfolded_backward against the fp64 backward oracle with
    the GPU's selections, every row (ragged tails, a query offset, d 64)."""
    layout, L, B, Hq, Hkv, d, q_begin = UNF[case]
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=700 + case, dtype="bf16")
    do = inputs.round_bf16(np.random.default_rng(800 + case).standard_normal((B, L, Hq, d), dtype=np.float32))
    q, do = q[:, q_begin:], do[:, q_begin:]
    sel, dq, dk, dv = _unfolded_forward_backward(layout, q, k, v, do, q_begin, grad_dtype)
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    rq, rk, rv, _, _ = GB.attend_backward(lay, tm, q, k, v, do, list(range(q_begin, L)), 1 / math.sqrt(d), sel)
    tag = f"unfolded case {case} {grad_dtype}"
    assert_grad_close(dq, rq, "dq " + tag)
    assert_grad_close(dk, rk, "dk " + tag)
    assert_grad_close(dv, rv, "dv " + tag)


def test_unfolded_backward_k16_workload_sampled():
    """The 3B-shape 32K workload with per-query top-16 unfolding: dq of sampled
    rows, and dk/dv of sampled raw keys far from the window's reach, which the
    oracle evaluates over every row that sees them (their window and the rows
    whose selection unfolds their chunk)."""
    w = configs.LLAMA3B_K16_PREFILL
    L = w.seq_len
    q, k, v = inputs.prefill_inputs(w, seed=21)
    do = inputs.round_bf16(np.random.default_rng(22).standard_normal((w.batch, L, w.hq, w.d), dtype=np.float32))
    sel, dq, dk, dv = _unfolded_forward_backward(w.layout, q, k, v, do, 0, torch.float32)
    lay = O.Layout.of(w.layout)
    tm = O.type_map(lay, L)
    scale = 1 / math.sqrt(w.d)
    rng = np.random.default_rng(23)
    rows = sorted(set(rng.integers(0, L, 5).tolist()) | {L - 1})
    rq, _, _, _, _ = GB.attend_backward(lay, tm, q[:, rows], k, v, do[:, rows], rows, scale, sel[:, :, rows])
    assert_grad_close(dq[:, rows], rq, "dq k16 rows")
    typ = np.asarray(tm.typ)
    raws = np.nonzero(typ == O.RAW)[0]
    for p in [int(x) for x in rng.choice(raws[(raws > 4000) & (raws < 30000)], 2, replace=False)]:
        chunk = int(tm.chunk[p])
        see = set(range(p, min(L, p + w.window)))
        see |= set(np.nonzero((sel[0] == chunk).any(axis=-1))[1].tolist())
        rr = sorted(see)
        _, rk, rv, _, _ = GB.attend_backward(lay, tm, q[:, rr], k, v, do[:, rr], rr, scale, sel[:, :, rr])
        assert_grad_close(dk[:, p], rk[:, p], f"dk raw key {p}")
        assert_grad_close(dv[:, p], rv[:, p], f"dv raw key {p}")
