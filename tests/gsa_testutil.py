"""Shared helpers of the parity tests (GPU path vs fp64 oracle).

Comparison protocol:
  * tables and tile lists: bit-exact;
  * selections: bit-exact, except rows whose oracle k-th / (k+1)-th score gap
    is below 1e-3, where the GPU set must be a valid near-top-k (every chosen
    score >= s_k - 1e-3, every unchosen score <= s_(k+1) + 1e-3);
  * attention outputs: the oracle is evaluated with the GPU's (validated)
    selection; max-abs error <= 1e-4 for fp32 inputs, <= 1e-2 for bf16 inputs
    on an fp32 output, plus half a bf16 ulp of the reference when the output
    itself is bf16.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import gsa_oracle as O

NEAR_TIE = 1e-3
TOL = {"f32": 1e-4, "bf16": 1e-2}
# Log-sum-exp is an auxiliary output the pages do not mention; the tolerances
# are the output tolerances' counterparts (1e-4 fp32, 1e-3 bf16).  The kernels
# form it from an fp32 sum of the unrounded probabilities.
LSE_TOL = {"f32": 1e-4, "bf16": 1e-3}


def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp of |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 1e-30)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def assert_close(got: np.ndarray, ref: np.ndarray, tol: float, bf16_out: bool = False, what=""):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    allow = tol + (bf16_half_ulp(ref) if bf16_out else 0.0)
    bad = err > allow
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    assert not bad.any(), (f"{what}: max-abs error {err.max():.3e} (allowed {tol:.1e}"
                           f"{' + half ulp' if bf16_out else ''}), {int(bad.sum())} elements over")
    return float(err.max())


def _valid_near_topk(scores: dict, chosen: list, k: int) -> bool:
    order = sorted(scores, key=lambda m: (-scores[m], m))
    want = min(k, len(order))
    if len(chosen) != want or len(set(chosen)) != want:
        return False
    if any(m not in scores for m in chosen):
        return False
    if want == len(order):
        return True
    sk, sk1 = scores[order[want - 1]], scores[order[want]]
    cs = set(chosen)
    return (all(scores[m] >= sk - NEAR_TIE for m in cs)
            and all(scores[m] <= sk1 + NEAR_TIE for m in scores if m not in cs))


def check_selection(lay: O.Layout, tm: O.TypeMap, q, k, positions, scale, gpu_sel, gpu_selg=None):
    """Validate GPU selections against the oracle (protocol above).

    ``q [B, Nq, Hq, d]``, ``k [B, L, Hkv, d]`` as numpy.  Returns the number
    of near-tie rows where the GPU differs (accepted)."""
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    accepted = 0
    if not lay.hierarchical:
        ref = O.select(lay, tm, q, k, positions, scale)
        diff = (gpu_sel != ref["sel"]).any(axis=-1)
        for b, h, r in zip(*np.nonzero(diff)):
            gap = ref["gap"][b, h, r]
            assert gap < NEAR_TIE, (f"selection differs at b={b} h={h} row={r} (gap {gap:.3e}): "
                                    f"gpu {gpu_sel[b, h, r].tolist()} oracle {ref['sel'][b, h, r].tolist()}")
            i = positions[r]
            s = O.gist_scores(q[b, r, h * G:(h + 1) * G], k[b, :, h], tm.chunk_gists,
                              O.chunk_candidates(lay, tm, i), scale)
            chosen = [int(x) for x in gpu_sel[b, h, r] if x >= 0]
            assert _valid_near_topk(s, chosen, lay.top_k), f"invalid near-top-k at {(b, h, r)}"
            assert list(gpu_sel[b, h, r][:len(chosen)]) == sorted(chosen)
            accepted += 1
        return accepted
    ref2 = O.select(lay, tm, q, k, positions, scale)
    diff2 = (gpu_selg != ref2["sel_groups"]).any(axis=-1)
    for b, h, r in zip(*np.nonzero(diff2)):
        gap = ref2["gap2"][b, h, r]
        assert gap < NEAR_TIE, f"group selection differs at {(b, h, r)} (gap {gap:.3e})"
        i = positions[r]
        s = O.gist_scores(q[b, r, h * G:(h + 1) * G], k[b, :, h], tm.group_gists,
                          O.group_candidates(lay, tm, i), scale)
        chosen = [int(x) for x in gpu_selg[b, h, r] if x >= 0]
        assert _valid_near_topk(s, chosen, lay.l2_top_k), f"invalid near-top-k groups at {(b, h, r)}"
        accepted += 1
    # level 1 given the GPU's groups
    ref1 = O.select(lay, tm, q, k, positions, scale, forced_groups=gpu_selg)
    diff1 = (gpu_sel != ref1["sel"]).any(axis=-1)
    for b, h, r in zip(*np.nonzero(diff1)):
        gap = ref1["gap"][b, h, r]
        assert gap < NEAR_TIE, f"chunk selection differs at {(b, h, r)} (gap {gap:.3e})"
        i = positions[r]
        gids = [int(x) for x in gpu_selg[b, h, r] if x >= 0]
        cands = [m for m, gr in enumerate(tm.chunk_group) if gr in gids
                 and len(tm.chunk_gists[m]) == lay.gists and tm.chunk_gists[m][-1] < i]
        s = O.gist_scores(q[b, r, h * G:(h + 1) * G], k[b, :, h], tm.chunk_gists, cands, scale)
        chosen = [int(x) for x in gpu_sel[b, h, r] if x >= 0]
        assert _valid_near_topk(s, chosen, lay.top_k), f"invalid near-top-k chunks at {(b, h, r)}"
        accepted += 1
    return accepted


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
