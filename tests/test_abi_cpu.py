"""CPU-side checks of the C ABI: the library loads, exports every function
that include/gsa.h declares, and its host-only calls and argument checks
behave as documented (no kernel is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import gist_token_block_amd as gsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsa.h")


def declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gsa_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gsa.LIB_PATH):
        from gist_token_block_amd import build
        build.build()
    return gsa.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gsa.h but not exported"
    assert set(gsa.EXPORTS) == set(names)


def test_status_strings(lib):
    assert lib.gsa_status_str(0) == b"GSA_OK"
    assert lib.gsa_status_str(1) == b"GSA_EINVAL"
    assert lib.gsa_status_str(2) == b"GSA_EUNSUPPORTED"
    assert lib.gsa_status_str(3) == b"GSA_EHIP"
    assert lib.gsa_status_str(4) == b"GSA_EHOST"


def test_table_dims_stream_tiles(lib):
    # 3B-shape fixed layout: 2 sink + 128 gist + 512 raw tiles of 64
    lay = dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0)
    nqt, nkt = gsa.table_dims(lay, 41088, 41088, 128, 64)
    assert (nqt, nkt) == (321, 2 + 128 + 512)
    # short last tiles are kept per stream
    lay = dict(n_sink=5, chunk_len=3, gists=1, window=4, top_k=0)
    nqt, nkt = gsa.table_dims(lay, 5 + 10 * 4 + 2, 47, 16, 4)
    assert nqt == 3
    assert nkt == 2 + 3 + 8   # sinks 5 -> 2, gists 10 -> 3, raws 32 -> 8
    lay2 = dict(n_sink=2, chunk_len=8, gists=1, window=4, top_k=4, l2_chunks=8, l2_gists=1,
                l2_top_k=2)
    _, nkt2 = gsa.table_dims(lay2, 2 + 3 * 73, 1, 1, 64)
    assert nkt2 == 1 + 1 + 1 + 3   # sinks | 3 level-2 gists | 24 gists | 192 raws


def test_score_columns_and_workspace(lib):
    lay = dict(n_sink=128, chunk_len=32, gists=1, window=128, top_k=16)
    assert gsa.score_columns(lay, 128 + 1024 * 33 + 1) == 1024
    assert gsa.decode_workspace_bytes(lay, 16, 32, 8, 128, 128 + 1024 * 33 + 1) > 0
    lay2 = dict(n_sink=128, chunk_len=8, gists=1, window=128, top_k=16, l2_chunks=8, l2_gists=1,
                l2_top_k=8)
    assert gsa.score_columns(lay2, 128 + 1024 * 73 + 1) == 1024


def test_prefill_tile(lib):
    import torch
    assert gsa.prefill_tile(torch.bfloat16, 128) == (128, 64)
    assert gsa.prefill_tile(torch.float32, 64) == (64, 64)


def test_invalid_arguments_rejected_before_launch(lib):
    L = gsa.make_layout
    bad = [dict(n_sink=-1, chunk_len=4), dict(n_sink=0, chunk_len=0), dict(chunk_len=4, gists=0),
           dict(chunk_len=4, window=-2), dict(chunk_len=4, top_k=-1),
           dict(chunk_len=4, l2_chunks=2, l2_gists=1, l2_top_k=0, top_k=1),
           dict(chunk_len=4, l2_gists=1)]
    a, b = ctypes.c_int32(), ctypes.c_int32()
    for d in bad:
        st = lib.gsa_table_dims(ctypes.byref(L(d)), 100, 10, 16, 16, ctypes.byref(a), ctypes.byref(b))
        assert st == gsa.GSA_EINVAL, d
        assert lib.gsa_last_error()
    good = L(dict(chunk_len=4, top_k=2))
    # build_layout: missing sel with top_k > 0, rows out of range, null outputs
    assert lib.gsa_build_layout(ctypes.byref(good), 50, 0, 50, 16, 16, None, None, 1, 1, 1, 1,
                                None) == gsa.GSA_EINVAL
    assert b"sel is required" in lib.gsa_last_error()
    assert lib.gsa_build_layout(ctypes.byref(good), 50, 40, 20, 16, 16, 1, None, 1, 1, 1, 1,
                                None) == gsa.GSA_EINVAL
    # score_select: misaligned pointer, unsupported head dim
    t = gsa.Tensor(8, gsa.GSA_BF16, 0, 0, 0, 0)
    assert lib.gsa_score_select(ctypes.byref(good), t, t, 1, 1, 1, 128, 50, 0, 1, 0.1, 16, None,
                                None, None) == gsa.GSA_EINVAL
    t16 = gsa.Tensor(16, gsa.GSA_BF16, 0, 0, 0, 0)
    assert lib.gsa_score_select(ctypes.byref(good), t16, t16, 1, 1, 1, 96, 50, 0, 1, 0.1, 16, None,
                                None, None) == gsa.GSA_EUNSUPPORTED
    # prefill: wrong tile shape for the MFMA path, non-positive scale
    fixed = L(dict(chunk_len=4, window=8))
    assert lib.gsa_attn_prefill(ctypes.byref(fixed), t16, t16, t16, t16, None, 1, 1, 1, 128, 50, 0,
                                50, None, None, 16, 16, 16, 64, 64, 0.1, None) == gsa.GSA_EINVAL
    assert lib.gsa_attn_prefill(ctypes.byref(fixed), t16, t16, t16, t16, None, 1, 1, 1, 128, 50, 0,
                                50, None, None, 16, 16, 16, 128, 64, 0.0, None) == gsa.GSA_EINVAL
    # decode: workspace too small, dtype mismatch
    dl = L(dict(n_sink=4, chunk_len=4, window=8, top_k=2))
    assert lib.gsa_attn_decode(ctypes.byref(dl), t16, t16, t16, t16, None, 1, 4, 1, 128, 50, 16,
                               None, 0.1, 16, 1, None) == gsa.GSA_EINVAL
    t32 = gsa.Tensor(16, gsa.GSA_F32, 0, 0, 0, 0)
    assert lib.gsa_attn_decode(ctypes.byref(dl), t32, t32, t32, t32, None, 1, 4, 1, 128, 50, 16,
                               None, 0.1, 16, 1 << 30, None) == gsa.GSA_EUNSUPPORTED


def test_compact_sizes(lib):
    """Slots = sinks + gist capacity + max(window, 1); gists counted as the
    layout places them (ratio 4 at 32K raw tokens: 8192 gists)."""
    lay = dict(n_sink=128, chunk_len=4, gists=1, window=128, top_k=0)
    assert gsa.compact_slots(lay, 8192) == 128 + 8192 + 128
    assert gsa.compact_gists(lay, 128 + 8192 * 5 + 1) == 8192
    assert gsa.compact_gists(lay, 128 + 3 * 5 + 4) == 3
    assert gsa.compact_gists(lay, 128 + 3 * 5 + 5) == 4
    assert gsa.compact_slots(dict(n_sink=0, chunk_len=3, gists=2, window=0, top_k=0), 5) == 0 + 5 + 1
    assert gsa.compact_slots(dict(n_sink=1, chunk_len=3, gists=1, window=4, top_k=1), 5) == -1


@pytest.mark.parametrize("n_bytes,block,seed", [(8192, 128, 0), (1000, 64, 1), (777, 100, 2), (128, 128, 3),
                                                (300, 1, 4)])
def test_gzip_block_flags_match_the_oracle(n_bytes, block, seed):
    """Host-only call: ratios bit-exact (integer length / block) and flags
    exact against the oracle on mixed synthetic bytes, ragged tails included."""
    from oracle import gzip_mask as gm
    from workloads import inputs
    x = inputs.mixed_bytes(3, n_bytes, max(block, 16), seed)
    ratio, flags = gsa.gzip_block_flags(x, block)
    for b in range(3):
        r = gm.block_ratios(x[b].tobytes(), block)
        np.testing.assert_array_equal(ratio[b].astype(np.float64), r.astype(np.float32).astype(np.float64))
        np.testing.assert_array_equal(flags[b].astype(bool), gm.literal_flags(r))


def test_block_mask_arguments_rejected_before_launch(lib):
    p = ctypes.c_void_p(16)
    # block not a multiple of the tile, q_begin misaligned, wrong block count, negative band
    assert lib.gsa_build_block_mask(p, 1, 8, 96, 1, 768, 0, 768, 128, 64, p, p, p, None) == gsa.GSA_EUNSUPPORTED
    assert lib.gsa_build_block_mask(p, 1, 6, 128, 1, 768, 64, 704, 128, 64, p, p, p, None) == gsa.GSA_EUNSUPPORTED
    assert lib.gsa_build_block_mask(p, 1, 5, 128, 1, 768, 0, 768, 128, 64, p, p, p, None) == gsa.GSA_EINVAL
    assert lib.gsa_build_block_mask(p, 1, 6, 128, -1, 768, 0, 768, 128, 64, p, p, p, None) == gsa.GSA_EINVAL
    assert lib.gsa_gzip_block_flags(None, 1, 10, 10, 4, None, p) == gsa.GSA_EINVAL
    t16 = gsa.Tensor(16, gsa.GSA_BF16, 0, 0, 0, 0)
    assert lib.gsa_attn_prefill_blockmask(t16, t16, t16, t16, None, 1, 1, 1, 64, 512, 0, 512, p, p, p, 64, 64,
                                          0.1, None) == gsa.GSA_EINVAL


def test_empty_query_range_is_a_no_op(lib):
    """q_len = 0: GSA_OK once the layout and the range are valid, with NULL
    tensors and outputs (nothing is launched, so this runs without a GPU);
    an invalid layout or range is still rejected."""
    L = gsa.make_layout
    sel_lay = L(dict(n_sink=4, chunk_len=4, window=8, top_k=2))
    fixed = L(dict(n_sink=4, chunk_len=4, window=8))
    null = gsa.Tensor(None, gsa.GSA_BF16, 0, 0, 0, 0)
    assert lib.gsa_build_layout(ctypes.byref(sel_lay), 50, 10, 0, 128, 64, None, None, 1, None, None, None,
                                None) == gsa.GSA_OK
    assert lib.gsa_score_select(ctypes.byref(sel_lay), null, null, 1, 2, 1, 128, 50, 10, 0, 0.1, None, None,
                                None, None) == gsa.GSA_OK
    assert lib.gsa_select_prefill(ctypes.byref(sel_lay), null, null, 1, 2, 1, 128, 50, 0, 0, 0.1, None,
                                  None) == gsa.GSA_OK
    assert lib.gsa_attn_prefill(ctypes.byref(fixed), null, null, null, null, None, 1, 2, 1, 128, 50, 50, 0,
                                None, None, None, None, None, 128, 64, 0.1, None) == gsa.GSA_OK
    assert lib.gsa_attn_prefill_unfolded(ctypes.byref(sel_lay), null, null, null, null, None, 1, 2, 1, 128, 50,
                                         0, 0, None, None, None, None, 128, 64, 0.1, None, 0, None) == gsa.GSA_OK
    assert lib.gsa_build_block_mask(None, 1, 1, 128, 2, 100, 0, 0, 128, 64, None, None, None,
                                    None) == gsa.GSA_OK
    # the range and the layout are still checked
    assert lib.gsa_attn_prefill(ctypes.byref(fixed), null, null, null, null, None, 1, 2, 1, 128, 50, 51, 0,
                                None, None, None, None, None, 128, 64, 0.1, None) == gsa.GSA_EINVAL
    bad = L(dict(n_sink=0, chunk_len=0))
    assert lib.gsa_build_layout(ctypes.byref(bad), 50, 0, 0, 128, 64, None, None, 1, None, None, None,
                                None) == gsa.GSA_EINVAL
