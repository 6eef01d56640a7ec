"""Pins of the backward oracle (oracle/gsa_backward.py) against facts other
than its own formulas: PyTorch autograd through a dense masked attention
built from the (separately pinned) visibility masks, central finite
differences of the pinned forward, and closed-form invariants of the softmax
derivative.

Source of the training setting: Forget, Then Recall ... Gist Sparse Attention
(abstract); UniGist summary (Approach, Experimental setup).
"""
import numpy as np
import pytest
import torch

from oracle import gsa_backward as GB
from oracle import gsa_oracle as O
from workloads import inputs


def _torch_grads(lay, tm, q, k, v, do, positions, scale, sel=None, selg=None):
    """Autograd of dense masked attention (fp64): the mask rows come from
    mask_row, the softmax and products from PyTorch."""
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    mask = np.zeros((B, Hkv, Nq, L), dtype=bool)
    for b in range(B):
        for h in range(Hkv):
            for r, i in enumerate(positions):
                s = () if sel is None else [m for m in sel[b, h, r] if m >= 0]
                g = () if selg is None else [m for m in selg[b, h, r] if m >= 0]
                mask[b, h, r] = O.mask_row(lay, tm, i, s, g)
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    qh = tq.permute(0, 2, 1, 3)                                       # [B, Hq, Nq, d]
    kh = tk.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)           # [B, Hq, L, d]
    vh = tv.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    m = torch.from_numpy(mask).repeat_interleave(G, dim=1)
    s = (qh @ kh.transpose(-1, -2)) * scale
    s = s.masked_fill(~m, float("-inf"))
    o = torch.softmax(s, dim=-1) @ vh
    (o * torch.from_numpy(do).permute(0, 2, 1, 3)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


CASES = [
    # layout, L, B, Hq, Hkv, d, q_begin, k
    (dict(n_sink=2, chunk_len=3, gists=1, window=4, top_k=0), 2 + 8 * 4 + 2, 2, 4, 2, 8, 0),
    (dict(n_sink=1, chunk_len=4, gists=2, window=3, top_k=2), 1 + 7 * 6 + 3, 1, 2, 1, 8, 5),
    (dict(n_sink=2, chunk_len=2, gists=1, window=2, top_k=2, l2_chunks=2, l2_gists=1, l2_top_k=1),
     2 + 6 * 7 + 2, 1, 4, 2, 6, 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_matches_autograd_of_masked_attention(case):
    ld, L, B, Hq, Hkv, d, q_begin = CASES[case]
    lay = O.Layout.of(ld)
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=100 + case, dtype="f32")
    do = np.random.default_rng(200 + case).standard_normal((B, L, Hq, d))
    pos = list(range(q_begin, L))
    q, do = q[:, q_begin:], do[:, q_begin:]
    scale = 0.35
    sel = selg = None
    if lay.top_k > 0:
        res = O.select(lay, tm, q, k, pos, scale)
        sel, selg = res["sel"], res.get("sel_groups")
    dq, dk, dv, o, lse = GB.attend_backward(lay, tm, q, k, v, do, pos, scale, sel, selg)
    tq, tk, tv = _torch_grads(lay, tm, q, k, v, do, pos, scale, sel, selg)
    np.testing.assert_allclose(dq, tq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv, rtol=0, atol=1e-12)
    fo, flse = O.attend(lay, tm, q, k, v, pos, scale, sel, selg)
    np.testing.assert_allclose(o, fo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, flse, rtol=0, atol=1e-12)


def test_backward_central_differences():
    """d(sum(dO * O)) / dx by central differences of the pinned forward."""
    lay = O.Layout(1, 2, 1, 2, 0)
    L, B, Hq, Hkv, d, scale = 1 + 3 * 3 + 1, 1, 2, 1, 3, 0.5
    tm = O.type_map(lay, L)
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal(s) for s in ((B, L, Hq, d), (B, L, Hkv, d), (B, L, Hkv, d)))
    do = rng.standard_normal((B, L, Hq, d))
    pos = list(range(L))

    def loss(q_, k_, v_):
        o, _ = O.attend(lay, tm, q_, k_, v_, pos, scale)
        return float((o * do).sum())

    dq, dk, dv, _, _ = GB.attend_backward(lay, tm, q, k, v, do, pos, scale)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(arr.shape):
            xp, xm = [a.copy() for a in (q, k, v)], [a.copy() for a in (q, k, v)]
            xp[which][idx] += eps
            xm[which][idx] -= eps
            num = (loss(*xp) - loss(*xm)) / (2 * eps)
            assert abs(num - grad[idx]) < 1e-7, (which, idx, num, grad[idx])


def test_softmax_derivative_invariants():
    """Per query the ds_j sum to zero, so the keys' dk sum to zero when one
    query row is differentiated; the probabilities sum to one, so the keys'
    dv sum to the rows' dO (over the KV group's heads)."""
    lay = O.Layout(2, 3, 1, 3, 0)
    L, B, Hq, Hkv, d = 2 + 6 * 4, 1, 3, 1, 5
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=5, dtype="f32")
    do = np.random.default_rng(6).standard_normal((B, L, Hq, d))
    for i in (0, 7, L - 1):
        _, dk, dv, _, _ = GB.attend_backward(lay, tm, q[:, i:i + 1], k, v, do[:, i:i + 1], [i], 0.4)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=1)[0, 0], do[0, i].sum(axis=0), atol=1e-12)


def test_single_visible_key():
    """Position 0 sees only itself: o = v_0, so dq = 0, dk_0 = 0, dv_0 = dO."""
    lay = O.Layout(1, 2, 1, 1, 0)
    L = 7
    tm = O.type_map(lay, L)
    q, k, v = inputs.random_qkv(1, L, 2, 2, 4, seed=3, dtype="f32")
    do = np.random.default_rng(4).standard_normal((1, 1, 2, 4))
    dq, dk, dv, o, _ = GB.attend_backward(lay, tm, q[:, :1], k, v, do, [0], 0.5)
    assert np.abs(dq).max() == 0.0
    assert np.abs(dk).max() == 0.0
    np.testing.assert_allclose(dv[0, 0], do[0, 0], atol=0)
    np.testing.assert_allclose(np.abs(dv[0, 1:]).max(), 0.0, atol=0)
    np.testing.assert_allclose(o[0, 0], v[0, 0].astype(np.float64), atol=0)
