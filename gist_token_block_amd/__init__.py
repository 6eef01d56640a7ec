"""Python binding of libgsa (gist-token sparse attention on gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/gsa.h``.  Torch provides device memory and the current
stream.  If ``libgsa.so`` is missing or no GPU is present the calls raise;
there is no fallback.

Layout dictionaries use the keys ``n_sink, chunk_len, gists, window, top_k,
l2_chunks, l2_gists, l2_top_k`` (see ``workloads.configs``).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsa.so")

GSA_OK, GSA_EINVAL, GSA_EUNSUPPORTED, GSA_EHIP, GSA_EHOST = 0, 1, 2, 3, 4
GSA_F32, GSA_BF16 = 0, 1


class GsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_sink", "chunk_len", "gists_per_chunk", "window", "top_k",
        "l2_chunks", "l2_gists", "l2_top_k")]


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


EXPORTS = ("gsa_table_dims", "gsa_build_layout", "gsa_score_select", "gsa_score_columns",
           "gsa_attn_prefill", "gsa_prefill_tile", "gsa_attn_decode", "gsa_attn_decode_noalloc",
           "gsa_decode_workspace_bytes", "gsa_decode_step", "gsa_decode_step_workspace_bytes",
           "gsa_compact_slots", "gsa_compact_gists", "gsa_compact_append", "gsa_compact_decode",
           "gsa_compact_decode_workspace_bytes", "gsa_select_prefill", "gsa_attn_prefill_unfolded",
           "gsa_prefill_unfolded_workspace_bytes", "gsa_gzip_block_flags", "gsa_build_block_mask",
           "gsa_attn_prefill_blockmask", "gsa_prefill_backward_workspace_bytes", "gsa_attn_prefill_backward",
           "gsa_attn_prefill_blockmask_backward", "gsa_prefill_unfolded_backward_workspace_bytes",
           "gsa_attn_prefill_unfolded_backward", "gsa_status_str", "gsa_last_error")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgsa.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gist_token_block_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, V = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    LP = P(Layout)
    lib.gsa_table_dims.argtypes = [LP, I32, I32, I32, I32, P(I32), P(I32)]
    lib.gsa_build_layout.argtypes = [LP, I32, I32, I32, I32, I32, V, V, I32, V, V, V, V]
    lib.gsa_score_select.argtypes = [LP, Tensor, Tensor, I32, I32, I32, I32, I32, I32, I32, F,
                                     V, V, V, V]
    lib.gsa_score_columns.argtypes = [LP, I32]
    lib.gsa_score_columns.restype = I32
    lib.gsa_attn_prefill.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32,
                                     I32, I32, I32, V, V, V, V, V, I32, I32, F, V]
    lib.gsa_prefill_tile.argtypes = [I32, I32, P(I32), P(I32)]
    lib.gsa_attn_decode.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32, I32,
                                    V, V, F, V, ctypes.c_size_t, V]
    lib.gsa_attn_decode_noalloc.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32,
                                            I32, V, V, F, V]
    lib.gsa_decode_workspace_bytes.argtypes = [LP, I32, I32, I32, I32, I32]
    lib.gsa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_decode_step.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32, I32, F,
                                    V, V, V, ctypes.c_size_t, V]
    lib.gsa_decode_step_workspace_bytes.argtypes = [LP, I32, I32, I32, I32, I32]
    lib.gsa_decode_step_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_compact_slots.argtypes = [LP, I32]
    lib.gsa_compact_slots.restype = I32
    lib.gsa_compact_gists.argtypes = [LP, I32]
    lib.gsa_compact_gists.restype = I32
    lib.gsa_compact_append.argtypes = [LP, Tensor, Tensor, I32, I32, I32, I32, I32, Tensor, Tensor, I32, V]
    lib.gsa_compact_decode.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32, I32, I32, F,
                                       V, ctypes.c_size_t, V]
    lib.gsa_compact_decode_workspace_bytes.argtypes = [LP, I32, I32, I32, I32, I32]
    lib.gsa_compact_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_select_prefill.argtypes = [LP, Tensor, Tensor, I32, I32, I32, I32, I32, I32, I32, F, V, V]
    lib.gsa_attn_prefill_unfolded.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32, I32,
                                              I32, I32, V, V, V, V, I32, I32, F, V, ctypes.c_size_t, V]
    lib.gsa_prefill_unfolded_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.gsa_prefill_unfolded_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_gzip_block_flags.argtypes = [V, I32, I64, I32, I32, V, V]
    lib.gsa_build_block_mask.argtypes = [V, I32, I32, I32, I32, I32, I32, I32, I32, I32, V, V, V, V]
    lib.gsa_attn_prefill_blockmask.argtypes = [Tensor, Tensor, Tensor, Tensor, V, I32, I32, I32, I32, I32, I32,
                                               I32, V, V, V, I32, I32, F, V]
    lib.gsa_prefill_backward_workspace_bytes.argtypes = [I32, I32, I32]
    lib.gsa_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_attn_prefill_backward.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, Tensor, V, Tensor, Tensor, Tensor,
                                              I32, I32, I32, I32, I32, I32, I32, V, V, V, V, V, I32, I32, F, V,
                                              ctypes.c_size_t, V]
    lib.gsa_attn_prefill_blockmask_backward.argtypes = [Tensor, Tensor, Tensor, Tensor, Tensor, V, Tensor, Tensor,
                                                        Tensor, I32, I32, I32, I32, I32, I32, I32, V, V, V, I32, I32,
                                                        F, V, ctypes.c_size_t, V]
    lib.gsa_prefill_unfolded_backward_workspace_bytes.argtypes = [LP, I32, I32, I32, I32, I32]
    lib.gsa_prefill_unfolded_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.gsa_attn_prefill_unfolded_backward.argtypes = [LP, Tensor, Tensor, Tensor, Tensor, Tensor, V, Tensor,
                                                       Tensor, Tensor, I32, I32, I32, I32, I32, I32, I32, V, V, V, V,
                                                       I32, I32, F, V, ctypes.c_size_t, V]
    lib.gsa_status_str.argtypes = [I32]
    lib.gsa_status_str.restype = ctypes.c_char_p
    lib.gsa_last_error.argtypes = []
    lib.gsa_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("gsa_score_columns", "gsa_decode_workspace_bytes", "gsa_status_str",
                        "gsa_last_error", "gsa_decode_step_workspace_bytes", "gsa_compact_slots",
                        "gsa_compact_gists", "gsa_compact_decode_workspace_bytes",
                        "gsa_prefill_unfolded_workspace_bytes", "gsa_prefill_backward_workspace_bytes",
                        "gsa_prefill_unfolded_backward_workspace_bytes"):
            getattr(lib, name).restype = I32
    _lib = lib
    return lib


def _check(status: int):
    if status != GSA_OK:
        msg = _lib.gsa_last_error().decode()
        raise GsaError(status, msg)


def make_layout(d: dict) -> Layout:
    return Layout(int(d.get("n_sink", 0)), int(d["chunk_len"]), int(d.get("gists", 1)),
                  int(d.get("window", 0)), int(d.get("top_k", 0)), int(d.get("l2_chunks", 0)),
                  int(d.get("l2_gists", 0)), int(d.get("l2_top_k", 0)))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GSA_F32
    if t.dtype == torch.bfloat16:
        return GSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensor(t: torch.Tensor, sb: int, st: int, sh: int) -> Tensor:
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    return Tensor(t.data_ptr(), _dt(t), 0, sb, st, sh)


def _bthd(t: torch.Tensor) -> Tensor:
    """[B, T, H, d] tensor."""
    return _tensor(t, t.stride(0), t.stride(1), t.stride(2))


def _bhtd(t: torch.Tensor) -> Tensor:
    """[B, H, T, d] tensor (decode cache)."""
    return _tensor(t, t.stride(0), t.stride(2), t.stride(1))


def _bhd(t: torch.Tensor) -> Tensor:
    """[B, H, d] tensor (one token)."""
    return _tensor(t, t.stride(0), 0, t.stride(1))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def is_hierarchical(layout: dict) -> bool:
    return int(layout.get("l2_chunks", 0)) > 0


def table_dims(layout: dict, seq_len: int, q_len: int, block_m: int, block_n: int):
    lib = load_library()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.gsa_table_dims(ctypes.byref(make_layout(layout)), seq_len, q_len, block_m, block_n,
                              ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def prefill_tile(dtype: torch.dtype, d: int):
    lib = load_library()
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.gsa_prefill_tile(GSA_BF16 if dtype == torch.bfloat16 else GSA_F32, d,
                                ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def build_layout(layout: dict, seq_len: int, q_begin: int, q_len: int, block_m: int, block_n: int,
                 sel=None, sel_groups=None, n_tables: int = 1, device="cuda", out=None):
    """Visibility table, per-row tile counts and row-padded tile lists."""
    lib = load_library()
    nqt, nkt = table_dims(layout, seq_len, q_len, block_m, block_n)
    if out is None:
        table = torch.empty((n_tables, nqt, nkt), dtype=torch.int8, device=device)
        cnt = torch.empty((n_tables, nqt), dtype=torch.int32, device=device)
        lst = torch.empty((n_tables, nqt, max(nkt, 1)), dtype=torch.int32, device=device)
    else:
        table, cnt, lst = out
    for t in (sel, sel_groups):
        if t is not None:
            assert t.dtype == torch.int32 and t.is_contiguous()
    _check(lib.gsa_build_layout(ctypes.byref(make_layout(layout)), seq_len, q_begin, q_len,
                                block_m, block_n, _ptr(sel), _ptr(sel_groups), n_tables,
                                table.data_ptr(), cnt.data_ptr(), lst.data_ptr(), _stream()))
    return table, cnt, lst


def score_columns(layout: dict, seq_len: int) -> int:
    return int(load_library().gsa_score_columns(ctypes.byref(make_layout(layout)), seq_len))


def score_select(layout: dict, q: torch.Tensor, k: torch.Tensor, seq_len: int, q_begin: int,
                 scale: float | None = None, cache_layout: bool = False, want_scores: bool = False,
                 out=None):
    """Selections for queries ``q [B, Nq, Hq, d]`` (or ``[B, Hq, d]``: one query).

    ``k`` is ``[B, L, Hkv, d]``, or ``[B, Hkv, L, d]`` with ``cache_layout``.
    Returns (sel, sel_groups or None, scores or None)."""
    lib = load_library()
    if q.dim() == 3:
        q = q.unsqueeze(1)
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[1] if cache_layout else k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kt = _bhtd(k) if cache_layout else _bthd(k)
    K1 = int(layout.get("top_k", 0))
    hier = is_hierarchical(layout)
    if out is None:
        sel = torch.empty((B, Hkv, Nq, K1), dtype=torch.int32, device=q.device)
        selg = (torch.empty((B, Hkv, Nq, int(layout["l2_top_k"])), dtype=torch.int32,
                            device=q.device) if hier else None)
    else:
        sel, selg = out
    scores = None
    if want_scores:
        scores = torch.empty((B, Hkv, Nq, max(score_columns(layout, seq_len), 1)),
                             dtype=torch.float32, device=q.device)
    _check(lib.gsa_score_select(ctypes.byref(make_layout(layout)), _bthd(q), kt, B, Hq, Hkv, d,
                                seq_len, q_begin, Nq, float(scale), sel.data_ptr(), _ptr(selg),
                                _ptr(scores), _stream()))
    return sel, selg, scores


def attn_prefill(layout: dict, q, k, v, tables, block_m: int, block_n: int, sel=None,
                 sel_groups=None, q_begin: int = 0, scale: float | None = None,
                 out_dtype=torch.float32, want_lse: bool = True, out=None):
    """Block-sparse prefill; ``q [B, Nq, Hq, d]``, ``k``/``v`` ``[B, L, Hkv, d]``.

    ``tables`` is the (table, tile_cnt, tile_list) triple of ``build_layout``."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        o = torch.empty((B, Nq, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    table, cnt, lst = tables
    _check(lib.gsa_attn_prefill(ctypes.byref(make_layout(layout)), _bthd(q), _bthd(k), _bthd(v),
                                _bthd(o), _ptr(lse), B, Hq, Hkv, d, L, q_begin, Nq, _ptr(sel),
                                _ptr(sel_groups), table.data_ptr(), cnt.data_ptr(),
                                lst.data_ptr(), block_m, block_n, float(scale), _stream()))
    return o, lse


def decode_workspace_bytes(layout: dict, B: int, Hq: int, Hkv: int, d: int, kv_len: int) -> int:
    return int(load_library().gsa_decode_workspace_bytes(ctypes.byref(make_layout(layout)), B, Hq,
                                                         Hkv, d, kv_len))


def attn_decode(layout: dict, q, k_cache, v_cache, sel=None, sel_groups=None,
                scale: float | None = None, out_dtype=torch.float32, want_lse: bool = True,
                workspace=None, out=None):
    """Split-K decode; ``q [B, Hq, d]``, caches ``[B, Hkv, kv_len, d]``."""
    lib = load_library()
    B, Hq, d = q.shape
    Hkv, kv_len = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = decode_workspace_bytes(layout, B, Hq, Hkv, d, kv_len)
    if workspace is None:   # zero-filled once: the kernel leaves its counters at zero
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        o = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    _check(lib.gsa_attn_decode(ctypes.byref(make_layout(layout)), _bhd(q), _bhtd(k_cache),
                               _bhtd(v_cache), _bhd(o), _ptr(lse), B, Hq, Hkv, d, kv_len,
                               _ptr(sel), _ptr(sel_groups), float(scale), workspace.data_ptr(),
                               workspace.numel(), _stream()))
    return o, lse


def attn_decode_noalloc(layout: dict, q, k_cache, v_cache, sel=None, sel_groups=None,
                        scale: float | None = None, out_dtype=torch.float32, want_lse: bool = True,
                        out=None):
    """``attn_decode`` on the library's fixed per-device scratch (no workspace)."""
    lib = load_library()
    B, Hq, d = q.shape
    Hkv, kv_len = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        o = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    _check(lib.gsa_attn_decode_noalloc(ctypes.byref(make_layout(layout)), _bhd(q), _bhtd(k_cache),
                                       _bhtd(v_cache), _bhd(o), _ptr(lse), B, Hq, Hkv, d, kv_len,
                                       _ptr(sel), _ptr(sel_groups), float(scale), _stream()))
    return o, lse


def decode_step_workspace_bytes(layout: dict, B: int, Hq: int, Hkv: int, d: int, kv_len: int) -> int:
    return int(load_library().gsa_decode_step_workspace_bytes(ctypes.byref(make_layout(layout)), B, Hq,
                                                              Hkv, d, kv_len))


def decode_step(layout: dict, q, k_cache, v_cache, scale: float | None = None, out_dtype=torch.float32,
                want_lse: bool = True, workspace=None, out=None):
    """Fused selection + decode; ``q [B, Hq, d]``, caches ``[B, Hkv, kv_len, d]``.

    Returns (o, lse or None, sel, sel_groups or None).  ``out`` is an optional
    (o, lse, sel, sel_groups) tuple of preallocated outputs."""
    lib = load_library()
    B, Hq, d = q.shape
    Hkv, kv_len = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = decode_step_workspace_bytes(layout, B, Hq, Hkv, d, kv_len)
    if workspace is None:   # zero-filled once: the kernels leave their counters at zero
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        o = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
        sel = torch.empty((B, Hkv, 1, int(layout.get("top_k", 0))), dtype=torch.int32, device=q.device)
        selg = (torch.empty((B, Hkv, 1, int(layout["l2_top_k"])), dtype=torch.int32, device=q.device)
                if is_hierarchical(layout) else None)
    else:
        o, lse, sel, selg = out
    _check(lib.gsa_decode_step(ctypes.byref(make_layout(layout)), _bhd(q), _bhtd(k_cache), _bhtd(v_cache),
                               _bhd(o), _ptr(lse), B, Hq, Hkv, d, kv_len, float(scale), sel.data_ptr(),
                               _ptr(selg), workspace.data_ptr(), workspace.numel(), _stream()))
    return o, lse, sel, selg


def compact_slots(layout: dict, gist_capacity: int) -> int:
    return int(load_library().gsa_compact_slots(ctypes.byref(make_layout(layout)), gist_capacity))


def compact_gists(layout: dict, seq_len: int) -> int:
    return int(load_library().gsa_compact_gists(ctypes.byref(make_layout(layout)), seq_len))


def compact_append(layout: dict, k_new, v_new, pos0: int, k_cache, v_cache, gist_capacity: int):
    """Append tokens ``k_new``/``v_new [B, n, Hkv, d]`` at positions
    ``[pos0, pos0 + n)`` to compact caches ``[B, Hkv, slots, d]``."""
    lib = load_library()
    B, n, Hkv, d = k_new.shape
    _check(lib.gsa_compact_append(ctypes.byref(make_layout(layout)), _bthd(k_new), _bthd(v_new), B, Hkv, d,
                                  pos0, n, _bhtd(k_cache), _bhtd(v_cache), gist_capacity, _stream()))


def compact_decode(layout: dict, q, k_cache, v_cache, pos: int, gist_capacity: int,
                   scale: float | None = None, out_dtype=torch.float32, want_lse: bool = True,
                   workspace=None, out=None):
    """Decode ``q [B, Hq, d]`` at position ``pos`` over compact caches."""
    lib = load_library()
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if workspace is None:
        need = int(lib.gsa_compact_decode_workspace_bytes(ctypes.byref(make_layout(layout)), B, Hq, Hkv, d, pos))
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        o = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    _check(lib.gsa_compact_decode(ctypes.byref(make_layout(layout)), _bhd(q), _bhtd(k_cache), _bhtd(v_cache),
                                  _bhd(o), _ptr(lse), B, Hq, Hkv, d, pos, gist_capacity, float(scale),
                                  workspace.data_ptr(), workspace.numel(), _stream()))
    return o, lse


def compact_decode_workspace_bytes(layout: dict, B: int, Hq: int, Hkv: int, d: int, pos: int) -> int:
    return int(load_library().gsa_compact_decode_workspace_bytes(ctypes.byref(make_layout(layout)), B, Hq, Hkv,
                                                                 d, pos))


def select_prefill(layout: dict, q, k, seq_len: int, q_begin: int = 0, scale: float | None = None, out=None):
    """Top-k chunks of every query row ``q [B, Nq, Hq, d]`` over keys
    ``k [B, L, Hkv, d]`` (single level, one gist per chunk); returns sel."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    sel = out if out is not None else torch.empty((B, Hkv, Nq, int(layout["top_k"])), dtype=torch.int32,
                                                  device=q.device)
    _check(lib.gsa_select_prefill(ctypes.byref(make_layout(layout)), _bthd(q), _bthd(k), B, Hq, Hkv, d, seq_len,
                                  q_begin, Nq, float(scale), sel.data_ptr(), _stream()))
    return sel


def prefill_unfolded_workspace_bytes(B: int, Hq: int, d: int, q_len: int) -> int:
    return int(load_library().gsa_prefill_unfolded_workspace_bytes(B, Hq, d, q_len))


def attn_prefill_unfolded(layout: dict, q, k, v, sel, fixed_tables, block_m: int, block_n: int, q_begin: int = 0,
                          scale: float | None = None, out_dtype=torch.float32, want_lse: bool = True,
                          workspace=None, out=None):
    """Prefill with selective unfolding: ``fixed_tables`` is the (table,
    tile_cnt, tile_list) of the same layout with top_k = 0."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(max(prefill_unfolded_workspace_bytes(B, Hq, d, Nq), 256), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        o = torch.empty((B, Nq, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    table, cnt, lst = fixed_tables
    _check(lib.gsa_attn_prefill_unfolded(ctypes.byref(make_layout(layout)), _bthd(q), _bthd(k), _bthd(v),
                                         _bthd(o), _ptr(lse), B, Hq, Hkv, d, L, q_begin, Nq, sel.data_ptr(),
                                         table.data_ptr(), cnt.data_ptr(), lst.data_ptr(), block_m, block_n,
                                         float(scale), workspace.data_ptr(), workspace.numel(), _stream()))
    return o, lse


def gzip_block_flags(data, block: int):
    """Ratios and literal flags of byte sequences on the host.

    ``data`` is a uint8 numpy array ``[B, n_bytes]`` (or one ``bytes``).
    Returns (ratio float32 [B, n_blocks], flags int8 [B, n_blocks])."""
    import numpy as np
    lib = load_library()
    if isinstance(data, (bytes, bytearray)):
        data = np.frombuffer(bytes(data), dtype=np.uint8)[None, :]
    data = np.ascontiguousarray(data, dtype=np.uint8)
    B, n = data.shape
    nb = -(-n // block)
    ratio = np.empty((B, nb), dtype=np.float32)
    flags = np.empty((B, nb), dtype=np.int8)
    _check(lib.gsa_gzip_block_flags(data.ctypes.data, B, n, n, block, ratio.ctypes.data, flags.ctypes.data))
    return ratio, flags


def build_block_mask(flags: torch.Tensor, block: int, w: int, seq_len: int, q_begin: int, q_len: int,
                     block_m: int, block_n: int, out=None):
    """Tile tables of the block mask: ``flags`` device int8 ``[B, n_blocks]``.
    Returns (table [B, nqt, nkt], tile_cnt [B, nqt], tile_list [B, nqt, nkt])."""
    lib = load_library()
    assert flags.dtype == torch.int8 and flags.is_contiguous() and flags.dim() == 2
    B, nb = flags.shape
    nqt = -(-q_len // block_m)
    nkt = -(-seq_len // block_n)
    if out is None:
        table = torch.empty((B, nqt, nkt), dtype=torch.int8, device=flags.device)
        cnt = torch.empty((B, nqt), dtype=torch.int32, device=flags.device)
        lst = torch.empty((B, nqt, max(nkt, 1)), dtype=torch.int32, device=flags.device)
    else:
        table, cnt, lst = out
    _check(lib.gsa_build_block_mask(flags.data_ptr(), B, nb, block, w, seq_len, q_begin, q_len, block_m, block_n,
                                    table.data_ptr(), cnt.data_ptr(), lst.data_ptr(), _stream()))
    return table, cnt, lst


def attn_prefill_blockmask(q, k, v, tables, block_m: int, block_n: int, q_begin: int = 0,
                           scale: float | None = None, out_dtype=torch.float32, want_lse: bool = True, out=None):
    """Prefill under a block mask; ``q [B, Nq, Hq, d]``, ``k``/``v`` ``[B, L, Hkv, d]``,
    ``tables`` from ``build_block_mask``."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        o = torch.empty((B, Nq, Hq, d), dtype=out_dtype, device=q.device)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    else:
        o, lse = out
    table, cnt, lst = tables
    _check(lib.gsa_attn_prefill_blockmask(_bthd(q), _bthd(k), _bthd(v), _bthd(o), _ptr(lse), B, Hq, Hkv, d, L,
                                          q_begin, Nq, table.data_ptr(), cnt.data_ptr(), lst.data_ptr(), block_m,
                                          block_n, float(scale), _stream()))
    return o, lse


def prefill_backward_workspace_bytes(B: int, Hq: int, q_len: int) -> int:
    return int(load_library().gsa_prefill_backward_workspace_bytes(B, Hq, q_len))


def prefill_unfolded_backward_workspace_bytes(layout: dict, B: int, Hq: int, Hkv: int, seq_len: int,
                                              q_len: int) -> int:
    return int(load_library().gsa_prefill_unfolded_backward_workspace_bytes(ctypes.byref(make_layout(layout)), B,
                                                                            Hq, Hkv, seq_len, q_len))


def attn_prefill_unfolded_backward(layout: dict, q, k, v, o, do, lse, sel, fixed_tables, block_m: int,
                                   block_n: int, q_begin: int = 0, scale: float | None = None,
                                   grad_dtype=torch.float32, workspace=None, out=None):
    """dq, dk, dv of attn_prefill_unfolded: ``fixed_tables`` are the fixed
    layout's (top_k = 0) tables, ``o``/``lse`` the unfolded forward's."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if workspace is None:
        need = prefill_unfolded_backward_workspace_bytes(layout, B, Hq, Hkv, L, Nq)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        dq = torch.empty((B, Nq, Hq, d), dtype=grad_dtype, device=q.device)
        dk = torch.empty((B, L, Hkv, d), dtype=grad_dtype, device=q.device)
        dv = torch.empty((B, L, Hkv, d), dtype=grad_dtype, device=q.device)
    else:
        dq, dk, dv = out
    assert lse.dtype == torch.float32 and lse.is_contiguous()
    table, cnt, lst = fixed_tables
    _check(lib.gsa_attn_prefill_unfolded_backward(
        ctypes.byref(make_layout(layout)), _bthd(q), _bthd(k), _bthd(v), _bthd(o), _bthd(do), lse.data_ptr(),
        _bthd(dq), _bthd(dk), _bthd(dv), B, Hq, Hkv, d, L, q_begin, Nq, sel.data_ptr(), table.data_ptr(),
        cnt.data_ptr(), lst.data_ptr(), block_m, block_n, float(scale), workspace.data_ptr(), workspace.numel(),
        _stream()))
    return dq, dk, dv


def attn_prefill_backward(layout, q, k, v, o, do, lse, tables, block_m: int, block_n: int, q_begin: int = 0,
                          scale: float | None = None, grad_dtype=torch.float32, workspace=None, out=None,
                          sel=None, sel_groups=None):
    """dq, dk, dv of the block-sparse prefill.  ``layout`` is a layout dict
    or the string "blockmask" (tables of build_block_mask).
    ``q``/``do``/``o`` ``[B, Nq, Hq, d]``, ``k``/``v`` ``[B, L, Hkv, d]``,
    ``lse [B, Hq, Nq]``, ``sel``/``sel_groups`` and ``tables`` from the forward."""
    lib = load_library()
    B, Nq, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(max(prefill_backward_workspace_bytes(B, Hq, Nq), 256), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        dq = torch.empty((B, Nq, Hq, d), dtype=grad_dtype, device=q.device)
        dk = torch.empty((B, L, Hkv, d), dtype=grad_dtype, device=q.device)
        dv = torch.empty((B, L, Hkv, d), dtype=grad_dtype, device=q.device)
    else:
        dq, dk, dv = out
    assert lse.dtype == torch.float32 and lse.is_contiguous()
    table, cnt, lst = tables
    head = (_bthd(q), _bthd(k), _bthd(v), _bthd(o), _bthd(do), lse.data_ptr(), _bthd(dq), _bthd(dk), _bthd(dv),
            B, Hq, Hkv, d, L, q_begin, Nq)
    tail = (table.data_ptr(), cnt.data_ptr(), lst.data_ptr(), block_m, block_n, float(scale), workspace.data_ptr(),
            workspace.numel(), _stream())
    if isinstance(layout, str):
        assert layout == "blockmask" and sel is None and sel_groups is None
        _check(lib.gsa_attn_prefill_blockmask_backward(*head, *tail))
    else:
        _check(lib.gsa_attn_prefill_backward(ctypes.byref(make_layout(layout)), *head, _ptr(sel), _ptr(sel_groups),
                                             *tail))
    return dq, dk, dv
