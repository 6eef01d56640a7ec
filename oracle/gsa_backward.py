"""Plain fp64 CPU oracle of the backward pass of gist-token sparse attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module; the library path never calls it and it
shares no code with the HIP kernels.

The pages train the sparse pattern end to end (Forget, Then Recall ... Gist
Sparse Attention, abstract; UniGist summary, Approach and Experimental setup,
which name forward and backward latency).  The backward of one query row is
the derivative of softmax attention over the row's visible keys -- the same
visibility as the forward (oracle.gsa_oracle.mask_row) -- written out:

    s_j  = scale * q . k_j              (j visible)
    p    = softmax(s)                   o = sum_j p_j v_j
    dp_j = dO . v_j                     delta = dO . o = sum_j p_j dp_j
    ds_j = p_j (dp_j - delta)
    dq   = scale * sum_j ds_j k_j
    dk_j += scale * ds_j q              dv_j += p_j dO

Keys collect over every query row and every query head of their KV group.
"""
import numpy as np

from .gsa_oracle import Layout, TypeMap, mask_row


def _row_sel(sel, b, h, r):
    if sel is None:
        return ()
    return [m for m in sel[b, h, r] if m >= 0]


def attend_backward(lay: Layout, tm: TypeMap, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    do: np.ndarray, positions, scale: float, sel=None, sel_groups=None):
    """Gradients of the sparse attention output with respect to q, k and v.

    ``q``/``do`` ``[B, Nq, Hq, d]`` with row r at ``positions[r]``; ``k``/``v``
    ``[B, L, Hkv, d]``.  Returns ``dq [B, Nq, Hq, d]``, ``dk``/``dv``
    ``[B, L, Hkv, d]`` and the forward's ``o`` and ``lse`` (fp64).
    """
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dq = np.zeros((B, Nq, Hq, d))
    dk = np.zeros((B, L, Hkv, d))
    dv = np.zeros((B, L, Hkv, d))
    o = np.zeros((B, Nq, Hq, d))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hkv):
            kh = k[b, :, h, :].astype(np.float64)
            vh = v[b, :, h, :].astype(np.float64)
            for r in range(Nq):
                vis = mask_row(lay, tm, positions[r], _row_sel(sel, b, h, r), _row_sel(sel_groups, b, h, r))
                idx = np.nonzero(vis)[0]
                kk, vv = kh[idx], vh[idx]
                for hq in range(h * G, (h + 1) * G):
                    qr = q[b, r, hq, :].astype(np.float64)
                    dor = do[b, r, hq, :].astype(np.float64)
                    s = (kk @ qr) * scale
                    mx = s.max()
                    ls = mx + np.log(np.exp(s - mx).sum())
                    p = np.exp(s - ls)
                    orow = p @ vv
                    dp = vv @ dor
                    delta = dor @ orow
                    ds = p * (dp - delta)
                    dq[b, r, hq, :] = scale * (ds @ kk)
                    dk[b, idx, h, :] += scale * np.outer(ds, qr)
                    dv[b, idx, h, :] += np.outer(p, dor)
                    o[b, r, hq, :] = orow
                    lse[b, hq, r] = ls
    return dq, dk, dv, o, lse
