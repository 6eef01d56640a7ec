"""GPU parity of the gzip-guided block-mask path (Gzip-guided sparse attention
page, Core equations): host flags (zlib), the tile table built on the GPU
(bit-exact against the oracle's codes of its token mask) and the prefill over
it (against fp64 masked attention).  Inputs: workloads.inputs.mixed_bytes and
random_qkv, seeded.
"""
import math

import numpy as np
import pytest
import torch

import gist_token_block_amd as gsa
from oracle import gzip_mask as gm
from workloads import configs, inputs

from gsa_testutil import LSE_TOL, TOL, assert_close, dev

pytestmark = pytest.mark.gpu


def _masks_and_flags(x, block, w, flags=None):
    if flags is None:
        flags = np.stack([gm.literal_flags(gm.block_ratios(x[b].tobytes(), block)) for b in range(x.shape[0])])
    masks = [gm.token_mask(gm.block_mask(flags[b].astype(bool), w), x.shape[1], block) for b in range(x.shape[0])]
    return masks, flags


def _check_tables(tables, masks, q_begin, q_len, bm, bn):
    table, cnt, lst = (t.cpu().numpy() for t in tables)
    for b, m in enumerate(masks):
        codes = gm.tile_codes(m, q_begin, q_len, bm, bn)
        np.testing.assert_array_equal(table[b], codes)
        for qt in range(codes.shape[0]):
            want = np.nonzero(codes[qt])[0]
            assert cnt[b, qt] == len(want)
            np.testing.assert_array_equal(lst[b, qt, :len(want)], want)


CASES = [
    # B, n_bytes, block, w, q_begin, bm, bn, seed
    (2, 1000, 128, 1, 0, 128, 64, 1),
    (3, 2048, 256, 0, 256, 128, 64, 2),
    (2, 700, 64, 2, 64, 64, 64, 3),
    (1, 8192, 128, 2, 0, 128, 64, 4),
]


@pytest.mark.parametrize("case", CASES)
def test_block_mask_table_matches_oracle(case):
    B, n, block, w, q_begin, bm, bn, seed = case
    x = inputs.mixed_bytes(B, n, block, seed)
    masks, _ = _masks_and_flags(x, block, w)
    _, flags = gsa.gzip_block_flags(x, block)
    tables = gsa.build_block_mask(torch.from_numpy(flags).to(dev()), block, w, n, q_begin, n - q_begin, bm, bn)
    torch.cuda.synchronize()
    _check_tables(tables, masks, q_begin, n - q_begin, bm, bn)


def _run_prefill(x, flags_np, block, w, q, k, v, bm, bn, q_begin, dtype, out_dtype):
    B, L = x.shape
    tq = torch.from_numpy(np.ascontiguousarray(q[:, q_begin:])).to(dev())
    tk, tv = torch.from_numpy(k).to(dev()), torch.from_numpy(v).to(dev())
    if dtype == "bf16":
        tq, tk, tv = tq.to(torch.bfloat16), tk.to(torch.bfloat16), tv.to(torch.bfloat16)
    tables = gsa.build_block_mask(torch.from_numpy(flags_np).to(dev()), block, w, L, q_begin, L - q_begin, bm, bn)
    o, lse = gsa.attn_prefill_blockmask(tq, tk, tv, tables, bm, bn, q_begin=q_begin,
                                        scale=1 / math.sqrt(q.shape[-1]), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return tables, o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("d,out_dtype", [(64, torch.float32), (128, torch.float32), (64, torch.bfloat16),
                                         (128, torch.bfloat16)])
def test_blockmask_prefill_bf16_matches_oracle(d, out_dtype):
    B, L, Hq, Hkv, block, w = 2, 700, 4, 2, 128, 1
    x = inputs.mixed_bytes(B, L, block, 10 + d)
    _, flags = gsa.gzip_block_flags(x, block)
    masks, _ = _masks_and_flags(x, block, w)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=20 + d, dtype="bf16")
    bm, bn = 128, 64
    tables, o, lse = _run_prefill(x, flags, block, w, q, k, v, bm, bn, 0, "bf16", out_dtype)
    _check_tables(tables, masks, 0, L, bm, bn)
    ro, rl = gm.attend_masked(q, k, v, masks, 1 / math.sqrt(d))
    assert_close(o, ro, TOL["bf16"], bf16_out=out_dtype == torch.bfloat16, what=f"o d={d}")
    assert_close(lse, rl, LSE_TOL["bf16"], what=f"lse d={d}")


def test_blockmask_prefill_f32_rowwave_with_offset():
    B, L, Hq, Hkv, d, block, w = 2, 600, 2, 1, 32, 64, 2
    x = inputs.mixed_bytes(B, L, block, 31)
    _, flags = gsa.gzip_block_flags(x, block)
    masks, _ = _masks_and_flags(x, block, w)
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=32, dtype="f32")
    q_begin = 128
    _, o, lse = _run_prefill(x, flags, block, w, q, k, v, 64, 64, q_begin, "f32", torch.float32)
    rows = list(range(q_begin, L))
    ro, rl = gm.attend_masked(q, k, v, masks, 1 / math.sqrt(d), rows=rows)
    assert_close(o, ro[:, q_begin:], TOL["f32"], what="o f32")
    assert_close(lse, rl[:, :, q_begin:], LSE_TOL["f32"], what="lse f32")


def test_all_literal_flags_give_causal_attention():
    B, L, Hq, Hkv, d, block = 1, 512, 2, 2, 64, 128
    x = inputs.mixed_bytes(B, L, block, 41)
    flags = np.ones((B, L // block), dtype=np.int8)
    masks, _ = _masks_and_flags(x, block, 0, flags=flags)
    assert (masks[0] == np.tril(np.ones((L, L), dtype=bool))).all()
    q, k, v = inputs.random_qkv(B, L, Hq, Hkv, d, seed=42, dtype="bf16")
    tables, o, lse = _run_prefill(x, flags, block, 0, q, k, v, 128, 64, 0, "bf16", torch.float32)
    _check_tables(tables, masks, 0, L, 128, 64)
    ro, rl = gm.attend_masked(q, k, v, masks, 1 / math.sqrt(d))
    assert_close(o, ro, TOL["bf16"], what="o causal")
    assert_close(lse, rl, LSE_TOL["bf16"], what="lse causal")


def test_workload_sampled_rows():
    wl = configs.GZIP_BLOCKMASK_PREFILL
    B, L = wl.batch, wl.n_bytes
    x = inputs.mixed_bytes(B, L, wl.block, 2026)
    _, flags = gsa.gzip_block_flags(x, wl.block)
    masks, oflags = _masks_and_flags(x, wl.block, wl.w)
    np.testing.assert_array_equal(flags.astype(bool), oflags)
    q, k, v = inputs.random_qkv(B, L, wl.hq, wl.hkv, wl.d, seed=2027, dtype="bf16")
    tables, o, lse = _run_prefill(x, flags, wl.block, wl.w, q, k, v, 128, 64, 0, "bf16", torch.bfloat16)
    _check_tables(tables, masks, 0, L, 128, 64)
    rng = np.random.default_rng(5)
    rows = sorted(set(rng.integers(0, L, 20).tolist()) | {0, 127, 128, L - 1})
    ro, rl = gm.attend_masked(q, k, v, masks, 1 / math.sqrt(wl.d), rows=rows)
    assert_close(o[:, rows], ro[:, rows], TOL["bf16"], bf16_out=True, what="o workload")
    assert_close(lse[:, :, rows], rl[:, :, rows], LSE_TOL["bf16"], what="lse workload")
