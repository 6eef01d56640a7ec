"""gsa_attn_decode_noalloc (fixed per-device scratch, no workspace) against
gsa_attn_decode (caller workspace): the same kernels on the same inputs, so the
outputs must agree exactly; two calls in a row, the second on a smaller input
(fewer sequences and KV heads, another layout), then the first again."""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from workloads import configs, inputs
from gsa_testutil import TOL, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _case(w, seed):
    x = inputs.decode_inputs(w, seed=seed)
    tq, tk, tv = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16")
    scale = 1 / math.sqrt(w.d)
    sel, selg, _ = gsa.score_select(w.layout, tq, tk, w.seq_len, w.seq_len - 1, scale, cache_layout=True)
    return w.layout, tq, tk, tv, sel, selg, scale


def _small():
    return configs.Workload(name="small", kind="decode", dtype="bf16", batch=3, hq=8, hkv=2, d=128,
                            n_sink=4, chunk_len=8, gists=1, window=16, top_k=5, n_chunks=70,
                            plant_chunks=5)


def _compare(case):
    layout, tq, tk, tv, sel, selg, scale = case
    ref_o, ref_lse = gsa.attn_decode(layout, tq, tk, tv, sel, selg, scale)
    o, lse = gsa.attn_decode_noalloc(layout, tq, tk, tv, sel, selg, scale)
    torch.cuda.synchronize()
    # the bar of the parity tests (bf16 inputs: 1e-2), and in fact bit-identical
    assert_close(o.cpu().numpy(), ref_o.cpu().numpy().astype(np.float64), TOL["bf16"], what="noalloc o")
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)


def test_noalloc_matches_workspace_decode_twice():
    big = _case(configs.SELECTIVE_DECODE, seed=17)
    small = _case(_small(), seed=18)
    _compare(big)
    _compare(small)     # second call, smaller input
    _compare(big)       # and back: the counters were left at zero


def test_noalloc_two_levels():
    _compare(_case(configs.HIER_DECODE, seed=19))


def test_noalloc_rejects_oversize():
    layout = dict(n_sink=4, chunk_len=8, gists=1, window=16, top_k=2)
    L = 4 + 9 * 10 + 1
    dev = torch.device("cuda:0")
    q = torch.zeros((20000, 8, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 1, L, 128), dtype=torch.bfloat16, device=dev).expand(20000, 1, L, 128)
    sel = torch.zeros((20000, 1, 1, 2), dtype=torch.int32, device=dev)
    with pytest.raises(gsa.GsaError) as e:
        gsa.attn_decode_noalloc(layout, q, kc, kc, sel, None)
    assert e.value.status == gsa.GSA_EUNSUPPORTED
