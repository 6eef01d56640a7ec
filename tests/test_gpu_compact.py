"""GPU parity of the compact cache (fixed layout, raw tokens outside the window
removed): tokens appended in pieces, then decode over the compact cache, against
the fp64 oracle over the full sequence (same visible set: sinks, every gist,
the window) and against gsa_attn_decode over the full cache."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gsa_oracle as O
from workloads import configs, inputs
from gsa_testutil import LSE_TOL, TOL, assert_close, dev, to_dev

pytestmark = pytest.mark.gpu


def _full(B, L, Hq, Hkv, d, seed):
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=seed, dtype="bf16")
    return q, k, v      # [B, L, H, d]


def _append_all(layout, k, v, pieces, cap):
    """Compact caches [B, Hkv, slots, d] filled by appending [0, L) in pieces."""
    B, L, Hkv, d = k.shape
    slots = gsa.compact_slots(layout, cap)
    kc = torch.full((B, Hkv, slots, d), float("nan"), dtype=torch.bfloat16, device=dev())
    vc = torch.full((B, Hkv, slots, d), float("nan"), dtype=torch.bfloat16, device=dev())
    tk, tv = to_dev(k, "bf16"), to_dev(v, "bf16")
    p0 = 0
    for n in pieces:
        gsa.compact_append(layout, tk[:, p0:p0 + n], tv[:, p0:p0 + n], p0, kc, vc, cap)
        p0 += n
    assert p0 == L
    return kc, vc


CASES = [
    # layout, L, B, Hq, Hkv, d, append pieces
    (dict(n_sink=4, chunk_len=4, gists=1, window=16, top_k=0), 4 + 60 * 5 + 3, 2, 8, 2, 128, [50, 1, 200, 56]),
    (dict(n_sink=0, chunk_len=3, gists=2, window=7, top_k=0), 70 * 5 + 2, 1, 4, 4, 64, [352]),
    (dict(n_sink=16, chunk_len=8, gists=1, window=300, top_k=0), 16 + 40 * 9, 2, 16, 1, 128, [100, 100, 100, 76]),
    (dict(n_sink=3, chunk_len=2, gists=1, window=1, top_k=0), 3 + 500 * 3 + 1, 1, 6, 2, 128, [1, 2, 3, 1498]),
    (dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0), 128 + 900 * 5 + 1, 2, 4, 1, 128, [4629]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_compact_decode_matches_oracle_and_full_cache(case):
    layout, L, B, Hq, Hkv, d, pieces = CASES[case]
    q, k, v = _full(B, L, Hq, Hkv, d, seed=90 + case)
    cap = gsa.compact_gists(layout, L) + 3
    kc, vc = _append_all(layout, k, v, pieces, cap)
    qd = q[:, L - 1]                        # the query at the last position
    tq = to_dev(qd, "bf16")
    scale = 1 / math.sqrt(d)
    o, lse = gsa.compact_decode(layout, tq, kc, vc, L - 1, cap, scale)
    torch.cuda.synchronize()
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    ref, ref_lse = O.attend(lay, tm, qd[:, None], k, v, [L - 1], scale)
    assert_close(o.cpu().numpy(), ref[:, 0], TOL["bf16"], what="compact decode")
    assert_close(lse.cpu().numpy(), ref_lse[:, :, 0], LSE_TOL["bf16"], what="compact decode lse")
    # the same visible set through the full cache
    kf = to_dev(np.ascontiguousarray(k.transpose(0, 2, 1, 3)), "bf16")
    vf = to_dev(np.ascontiguousarray(v.transpose(0, 2, 1, 3)), "bf16")
    of, _ = gsa.attn_decode(layout, tq, kf, vf, None, None, scale)
    torch.cuda.synchronize()
    assert np.abs(o.cpu().numpy() - of.cpu().numpy()).max() <= 1e-2


def test_compact_incremental_decode_loop():
    """Token-by-token generation: append one token, decode it, for 40 steps
    crossing several chunks and ring wrap-arounds."""
    layout = dict(n_sink=2, chunk_len=3, gists=1, window=6, top_k=0)
    L = 2 + 30 * 4
    B, Hq, Hkv, d = 2, 4, 2, 64
    q, k, v = _full(B, L, Hq, Hkv, d, seed=7)
    cap = gsa.compact_gists(layout, L)
    start = L - 40
    kc, vc = _append_all(layout, k[:, :start], v[:, :start], [start], cap)
    tk, tv = to_dev(k, "bf16"), to_dev(v, "bf16")
    lay = O.Layout.of(layout)
    tm = O.type_map(lay, L)
    scale = 0.2
    for p in range(start, L):
        gsa.compact_append(layout, tk[:, p:p + 1], tv[:, p:p + 1], p, kc, vc, cap)
        o, _ = gsa.compact_decode(layout, to_dev(q[:, p], "bf16"), kc, vc, p, cap, scale)
        torch.cuda.synchronize()
        ref, _ = O.attend(lay, tm, q[:, p:p + 1], k, v, [p], scale)
        assert_close(o.cpu().numpy(), ref[:, 0], TOL["bf16"], what=f"step {p}")


def test_compact_workload_shape_two_sequences():
    """The compact-decode workload's layout and head shape (32K raw tokens,
    ratio 4), two sequences; every head checked against the oracle."""
    w = configs.COMPACT_DECODE
    L = w.seq_len
    B = 2
    q, k, v = _full(B, L, w.hq, w.hkv, w.d, seed=3)
    cap = gsa.compact_gists(w.layout, L)
    kc, vc = _append_all(w.layout, k, v, [L - 1000, 1000], cap)
    assert gsa.compact_slots(w.layout, cap) == 128 + 8192 + 128
    scale = 1 / math.sqrt(w.d)
    o, lse = gsa.compact_decode(w.layout, to_dev(q[:, L - 1], "bf16"), kc, vc, L - 1, cap, scale)
    torch.cuda.synchronize()
    lay = O.Layout.of(w.layout)
    tm = O.type_map(lay, L)
    ref, ref_lse = O.attend(lay, tm, q[:, L - 1:L], k, v, [L - 1], scale)
    assert_close(o.cpu().numpy(), ref[:, 0], TOL["bf16"], what="compact workload")
    assert_close(lse.cpu().numpy(), ref_lse[:, :, 0], LSE_TOL["bf16"], what="compact workload lse")


def test_compact_rejects_unfolding_and_overflow():
    lay_k = dict(n_sink=2, chunk_len=4, gists=1, window=8, top_k=2)
    assert gsa.compact_slots(lay_k, 10) == -1
    layout = dict(n_sink=2, chunk_len=4, gists=1, window=8, top_k=0)
    L = 2 + 10 * 5
    q, k, v = _full(1, L, 2, 1, 64, seed=1)
    kc = torch.zeros((1, 1, gsa.compact_slots(layout, 3), 64), dtype=torch.bfloat16, device=dev())
    with pytest.raises(gsa.GsaError) as e:
        gsa.compact_append(layout, to_dev(k, "bf16"), to_dev(v, "bf16"), 0, kc, kc, 3)
    assert e.value.status == gsa.GSA_EINVAL
