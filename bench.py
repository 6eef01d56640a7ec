"""Benchmark of the gist-token sparse attention hot path on one MI355X.

Headline: block-sparse prefill of the Llama-3.2-3B attention shape at 32K raw
tokens (24 query / 8 KV heads, d=128, ratio 4: 1 gist after every 4 raw
tokens, 128 sinks, window 128, fixed layout k=0), bf16.  One step = build the
block-visibility table + run the prefill over it.  ``value`` is TFLOP/s on the
visible tiles (4 d x cells of the non-empty 128x64 tiles x batch x query heads,
per step time).  The same line carries:
  * ``roofline``: the prefill kernel's algorithmic TFLOP/s (4 d x visible pairs
    x batch x query heads, per kernel launch timed with HIP events on its
    stream) against the bf16 MFMA peak, and its counter-measured HBM bytes;
  * ``prefill``: the Llama-3.1-8B-shape 32K fixed-layout prefill, measured the
    same way;
  * ``decode``: the selective-unfolding and two-level decode workloads, one
    step = the fused selection + attention (gsa_decode_step), as GB/s of unique
    visible K/V bytes (+ q, o, indices) against HBM peak; the separate
    score_select + attn_decode calls are timed beside it;
  * ``cpu_baseline``: the fp64 oracle timed on the host cores on a sample of
    the headline workload, and on the full decode workloads.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-decode] [--no-cpu]
    python bench.py --profile-pass [--pass-workload NAME]   # short pass for rocprofv3 counter runs
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "sparse-attn TFLOP/s (32K prefill) & decode GB/s; % of MI355X roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_llama3b_32k_traffic.txt")
CSRC = os.path.join(ROOT, "gist_token_block_amd", "csrc")


# ---------------------------------------------------------------- closed forms (accounting)
def _counts(S, c, g, x):
    """(gists, raws) at positions < x for an array x (single level)."""
    P = c + g
    y = np.maximum(0, x - S)
    f, r = y // P, y % P
    return g * f + np.maximum(0, r - c), c * f + np.minimum(r, c)


def fixed_layout_edges(w, rows=None) -> int:
    """Visible (query, key) pairs per (batch, head) of a k=0 layout."""
    S, c, g, W1 = w.n_sink, w.chunk_len, w.gists, max(w.window, 1)
    i = np.arange(w.seq_len, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    lo = np.maximum(0, i - W1 + 1)
    gl, _ = _counts(S, c, g, lo)
    return int(((i - lo + 1) + np.minimum(S, lo) + gl).sum())


def visible_tile_cells(w, table: np.ndarray, bm: int, bn: int) -> int:
    """Cells of the non-empty tiles of one table (real extents)."""
    S, c, g, L = w.n_sink, w.chunk_len, w.gists, w.seq_len
    ng, nr = _counts(S, c, g, np.array([L]))
    widths = []
    for n in (min(S, L), int(ng[0]), int(nr[0])):
        widths += [min(bn, n - s) for s in range(0, n, bn)]
    widths = np.array(widths, dtype=np.int64)
    heights = np.array([min(bm, L - s) for s in range(0, L, bm)], dtype=np.int64)
    ne = table > 0
    return int((heights[:, None] * widths[None, :] * ne).sum())


def decode_unique_bytes(w, sel: np.ndarray, selg) -> tuple:
    """(unique visible rows over all (batch, KV head), bytes) of one decode step:
    each visible K and V row once, plus q, o and the selection indices."""
    rows = 0
    S, c, g, W1 = w.n_sink, w.chunk_len, w.gists, max(w.window, 1)
    L = w.seq_len
    i = L - 1
    lo = max(0, i - W1 + 1)
    P = c + g
    for bb in range(w.batch):
        for h in range(w.hkv):
            if not w.hierarchical:
                n_g = g * ((lo - S) // P) + max(0, (lo - S) % P - c)
                starts = [S + m * P for m in sel[bb, h, 0] if m >= 0]
            else:
                G2, g2 = w.l2_chunks, w.l2_gists
                P2 = G2 * P + g2
                y = lo - S
                n_g = g2 * (y // P2) + max(0, y % P2 - G2 * P)
                for gr in selg[bb, h, 0]:
                    if gr >= 0:
                        n_g += sum(min(max(lo - (S + gr * P2 + j * P + c), 0), g) for j in range(G2))
                starts = [S + (m // G2) * P2 + (m % G2) * P for m in sel[bb, h, 0] if m >= 0]
            rows += min(S, lo) + n_g + (i - lo + 1) + sum(min(max(lo - s0, 0), c) for s0 in starts)
    nbytes = rows * 2 * w.d * 2 + w.batch * w.hq * w.d * 2 * 2 + sel.nbytes + (0 if selg is None else selg.nbytes)
    return rows, int(nbytes)


def source_hash(files=None) -> str:
    h = hashlib.sha256()
    names = files or sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))
    for f in names:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or None
    if the kernel changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sha") != source_hash(["prefill_mfma.hip", "gsa_internal.h"]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_info() -> dict:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


# ---------------------------------------------------------------- oracle baseline
_POOL_ARGS = {}


def _oracle_worker(h):
    from oracle import gsa_oracle as O
    a = _POOL_ARGS
    t0 = time.perf_counter()
    O.attend(a["lay"], a["tm"], a["q"][:, :, h * a["G"]:(h + 1) * a["G"]], a["k"][:, :, h:h + 1],
             a["v"][:, :, h:h + 1], a["pos"], a["scale"], rows=a["rows"])
    return time.perf_counter() - t0


def cpu_baseline(w, q, k, v, rows_per_head: int):
    """The fp64 oracle on a sample of query rows (all heads), one process per
    KV head with single-threaded BLAS; rate in the headline's algorithmic
    FLOP/s."""
    import multiprocessing as mp
    from oracle import gsa_oracle as O
    lay = O.Layout.of(w.layout)
    tm = O.type_map(lay, w.seq_len)
    rows = np.linspace(0, w.seq_len - 1, rows_per_head).astype(int).tolist()
    flops = 4.0 * w.d * fixed_layout_edges(w, rows) * w.batch * w.hq
    _POOL_ARGS.update(lay=lay, tm=tm, q=q, k=k, v=v, G=w.hq // w.hkv, pos=list(range(w.seq_len)),
                      scale=1 / math.sqrt(w.d), rows=rows)
    from threadpoolctl import threadpool_limits
    info = host_info()
    workers = max(1, min(w.hkv, info["usable_cpus"], 16))
    ctx = mp.get_context("fork")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            pool.map(_oracle_worker, range(w.hkv))
        dt = time.perf_counter() - t0
    out = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": f"{len(rows)} query rows spread over the {w.seq_len} positions x all {w.hq} heads "
                     f"(batch {w.batch}) of {w.name}, fp64 numpy, {workers} processes x 1 BLAS thread "
                     f"(one per KV head), {dt:.1f} s wall"}
    out.update(info)
    return out


def cpu_baseline_decode(w):
    """The fp64 oracle (selection + attention) on one full decode step, serial."""
    from oracle import gsa_oracle as O
    from workloads import inputs
    x = inputs.decode_inputs(w, seed=11)
    lay = O.Layout.of(w.layout)
    L = w.seq_len
    scale = 1 / math.sqrt(w.d)
    kk = np.ascontiguousarray(x["k"].transpose(0, 2, 1, 3))
    vv = np.ascontiguousarray(x["v"].transpose(0, 2, 1, 3))
    q = x["q"][:, None]
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        tm = O.type_map(lay, L)
        res = O.select(lay, tm, q, kk, [L - 1], scale)
        O.attend(lay, tm, q, kk, vv, [L - 1], scale, res["sel"], res.get("sel_groups"))
        dt = time.perf_counter() - t0
    _, nbytes = decode_unique_bytes(w, res["sel"], res.get("sel_groups"))
    return {"workload": w.name, "value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"one full decode step (all {w.batch} x {w.hkv} groups: selection + attention), "
                      "fp64 numpy, 1 process x 1 BLAS thread"}


# ---------------------------------------------------------------- GPU legs
def run_prefill(w, args, torch, gsa, q, k, v):
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    bm, bn = gsa.prefill_tile(torch.bfloat16, w.d)
    nqt, nkt = gsa.table_dims(w.layout, w.seq_len, w.seq_len, bm, bn)
    tables = (torch.empty((1, nqt, nkt), dtype=torch.int8, device=dev),
              torch.empty((1, nqt), dtype=torch.int32, device=dev),
              torch.empty((1, nqt, nkt), dtype=torch.int32, device=dev))
    o = torch.empty((w.batch, w.seq_len, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    scale = 1 / math.sqrt(w.d)

    def step(ev=None):
        gsa.build_layout(w.layout, w.seq_len, 0, w.seq_len, bm, bn, out=tables)
        if ev is not None:
            ev[0].record()
        gsa.attn_prefill(w.layout, tq, tk, tv, tables, bm, bn, scale=scale, out=(o, None))
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    table = tables[0][0].cpu().numpy()
    step_ms = wall / args.steps * 1e3
    alg = 4.0 * w.d * fixed_layout_edges(w) * w.batch * w.hq
    tile = 4.0 * w.d * visible_tile_cells(w, table, bm, bn) * w.batch * w.hq
    del tq, tk, tv, o
    return {"workload": w.name, "ms_per_step": round(step_ms, 4), "kernel_ms": round(kern_ms, 4),
            "tflops_visible_tile": round(tile / (step_ms * 1e-3) / 1e12, 2),
            "tflops_algorithmic": round(alg / (kern_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(alg / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flops": alg, "visible_tile_flops": tile, "tile": [bm, bn],
            "tile_fill": round(alg / tile, 4)}


def run_backward(w, args, torch, gsa, q, k, v):
    """Prefill backward of a fixed layout: one forward (untimed) for O and
    the log-sum-exp, then one step = gsa_attn_prefill_backward (k_bwd_dq, which
    also forms D = rowsum(dO * O), then k_bwd_dkdv).  Algorithmic FLOPs per
    visible (query head, key) pair: 10 d (S recomputed once, dP, dV, dK, dQ);
    the kernels execute 14 d (S and dP are formed in both)."""
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    tdo = torch.randn(tq.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    bm, bn = gsa.prefill_tile(torch.bfloat16, w.d)
    tables = gsa.build_layout(w.layout, w.seq_len, 0, w.seq_len, bm, bn, device=dev)
    scale = 1 / math.sqrt(w.d)
    o, lse = gsa.attn_prefill(w.layout, tq, tk, tv, tables, bm, bn, scale=scale, out_dtype=torch.bfloat16)
    grads = (torch.empty(tq.shape, dtype=torch.bfloat16, device=dev),
             torch.empty(tk.shape, dtype=torch.bfloat16, device=dev),
             torch.empty(tv.shape, dtype=torch.bfloat16, device=dev))
    ws = torch.empty(gsa.prefill_backward_workspace_bytes(w.batch, w.hq, w.seq_len), dtype=torch.uint8, device=dev)

    def step():
        gsa.attn_prefill_backward(w.layout, tq, tk, tv, o, tdo, lse, tables, bm, bn, scale=scale, workspace=ws,
                                  out=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(5, args.steps // 2)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    kern_ms = ev[0].elapsed_time(ev[1]) / steps
    edges = fixed_layout_edges(w) * w.batch * w.hq
    alg = 10.0 * w.d * edges
    del tq, tk, tv, tdo, o, lse, grads, ws
    return {"workload": w.name + " (backward)", "ms_per_step": round(wall, 4), "kernel_ms": round(kern_ms, 4),
            "algorithmic_flops": alg, "executed_mfma_flops_per_pair": 14 * w.d,
            "tflops_algorithmic": round(alg / (kern_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(alg / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": "k_bwd_dq (also D) + k_bwd_dkdv; bf16 in, bf16 grads"}


def run_unfolded_backward(w, args, torch, gsa, q, k, v):
    """Backward of the selective-unfolding prefill: one forward (untimed:
    gsa_select_prefill, the fixed table, gsa_attn_prefill_unfolded with the
    log-sum-exp), then one step = gsa_attn_prefill_unfolded_backward (the fixed
    part's k_bwd_dq and k_bwd_dkdv, then the unfolded keys' share: dq per query
    row, the per-chunk lists, dk/dv per chunk).  Algorithmic FLOPs: 10 d per
    visible (query head, key) pair, unfolded pairs included."""
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    tdo = torch.randn(tq.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    bm, bn = gsa.prefill_tile(torch.bfloat16, w.d)
    scale = 1 / math.sqrt(w.d)
    sel = gsa.select_prefill(w.layout, tq, tk, w.seq_len, 0, scale)
    fixed = gsa.build_layout(dict(w.layout, top_k=0), w.seq_len, 0, w.seq_len, bm, bn, device=dev)
    o, lse = gsa.attn_prefill_unfolded(w.layout, tq, tk, tv, sel, fixed, bm, bn, 0, scale, out_dtype=torch.bfloat16)
    grads = (torch.empty(tq.shape, dtype=torch.bfloat16, device=dev),
             torch.empty(tk.shape, dtype=torch.bfloat16, device=dev),
             torch.empty(tv.shape, dtype=torch.bfloat16, device=dev))
    ws = torch.empty(gsa.prefill_unfolded_backward_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.seq_len,
                                                                   w.seq_len), dtype=torch.uint8, device=dev)

    def step():
        gsa.attn_prefill_unfolded_backward(w.layout, tq, tk, tv, o, tdo, lse, sel, fixed, bm, bn, 0, scale,
                                           workspace=ws, out=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(5, args.steps // 2)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    kern_ms = ev[0].elapsed_time(ev[1]) / steps
    alg = 10.0 * w.d * unfolded_edges(w, sel.cpu().numpy()) * (w.hq // w.hkv)
    del tq, tk, tv, tdo, o, lse, grads, ws, sel
    return {"workload": w.name + " (backward)", "ms_per_step": round(wall, 4), "kernel_ms": round(kern_ms, 4),
            "algorithmic_flops": alg, "tflops_algorithmic": round(alg / (kern_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(alg / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": "k_bwd_dq + k_unfold_bwd_q; k_bwd_dkdv + per-chunk lists + k_unfold_bwd_kv; bf16 grads"}


def run_decode(w, args, torch, gsa, copies=4):
    """One decode step = the fused selection + attention (gsa_decode_step);
    caches rotate over `copies` independent buffers so the visible rows are not
    served from the 256 MB Infinity Cache of a previous step.  The separate
    score_select + attn_decode calls are timed the same way for comparison."""
    from workloads import inputs
    dev = torch.device("cuda:0")
    x = inputs.decode_inputs(w, seed=11)
    tq = torch.from_numpy(x["q"]).to(dev).to(torch.bfloat16)
    kc0 = torch.from_numpy(x["k"]).to(dev).to(torch.bfloat16)
    vc0 = torch.from_numpy(x["v"]).to(dev).to(torch.bfloat16)
    del x
    caches = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(copies - 1)]
    L, scale = w.seq_len, 1 / math.sqrt(w.d)
    sel = torch.empty((w.batch, w.hkv, 1, w.top_k), dtype=torch.int32, device=dev)
    selg = (torch.empty((w.batch, w.hkv, 1, w.l2_top_k), dtype=torch.int32, device=dev)
            if w.hierarchical else None)
    o = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    ws_step = torch.zeros(gsa.decode_step_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L),
                          dtype=torch.uint8, device=dev)
    ws_dec = torch.zeros(gsa.decode_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L),
                         dtype=torch.uint8, device=dev)

    def fused(s):
        kc, vc = caches[s % copies]
        gsa.decode_step(w.layout, tq, kc, vc, scale, workspace=ws_step, out=(o, None, sel, selg))

    def separate(s):
        kc, vc = caches[s % copies]
        gsa.score_select(w.layout, tq, kc, L, L - 1, scale, cache_layout=True, out=(sel, selg))
        gsa.attn_decode(w.layout, tq, kc, vc, sel, selg, scale, workspace=ws_dec, out=(o, None))

    def timed(fn):
        """Per-step GPU time: one step per cache copy captured in a HIP graph
        and replayed, so the host's per-call launch cost (tens of us from
        Python) stays out of a ~40 us step."""
        for s in range(args.warmup):
            fn(s)
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(graph, stream=st):
                for s in range(copies):
                    fn(s)
        torch.cuda.current_stream().wait_stream(st)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, max(args.steps, 20) // copies)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * copies)

    ms_sep = timed(separate)
    ms = timed(fused)
    sl = sel.cpu().numpy()
    sg = selg.cpu().numpy() if selg is not None else None
    rows, nbytes = decode_unique_bytes(w, sl, sg)
    return {"workload": w.name, "ms_per_step": round(ms, 5),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "unique_bytes": nbytes,
            "visible_rows_per_group": round(float(rows) / (w.batch * w.hkv), 2),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels": "gsa_decode_step (k_step_a + k_step_b)", "cache_copies": copies,
            "timing": "HIP graph of one step per cache copy, replayed; events on the replay stream",
            "separate_calls_ms_per_step": round(ms_sep, 5)}


def unfolded_edges(w, sel: np.ndarray) -> int:
    """Visible pairs summed over (batch, KV head) of a single-level layout with
    the given selection [B, Hkv, L, k]: the fixed part per row plus the raws of
    each chosen chunk before the row's window."""
    S, c, g, W1, L = w.n_sink, w.chunk_len, w.gists, max(w.window, 1), w.seq_len
    P = c + g
    i = np.arange(L, dtype=np.int64)
    lo = np.maximum(0, i - W1 + 1)
    base = fixed_layout_edges(w)
    st = S + sel.astype(np.int64) * P
    extra = np.clip(lo[None, None, :, None] - st, 0, c)
    extra = np.where(sel >= 0, extra, 0)
    return int(base * sel.shape[0] * sel.shape[1] + extra.sum())


def run_unfolded(w, args, torch, gsa, q, k, v):
    """Selective-unfolding prefill: one step = gsa_select_prefill + the fixed
    part's table + gsa_attn_prefill_unfolded (unfold kernel, then the MFMA
    prefill starting from its partials)."""
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev).to(torch.bfloat16) for x in (q, k, v))
    bm, bn = gsa.prefill_tile(torch.bfloat16, w.d)
    fixed = dict(w.layout, top_k=0)
    nqt, nkt = gsa.table_dims(fixed, w.seq_len, w.seq_len, bm, bn)
    tables = (torch.empty((1, nqt, nkt), dtype=torch.int8, device=dev),
              torch.empty((1, nqt), dtype=torch.int32, device=dev),
              torch.empty((1, nqt, nkt), dtype=torch.int32, device=dev))
    sel = torch.empty((w.batch, w.hkv, w.seq_len, w.top_k), dtype=torch.int32, device=dev)
    o = torch.empty((w.batch, w.seq_len, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gsa.prefill_unfolded_workspace_bytes(w.batch, w.hq, w.d, w.seq_len), dtype=torch.uint8,
                     device=dev)
    scale = 1 / math.sqrt(w.d)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gsa.select_prefill(w.layout, tq, tk, w.seq_len, 0, scale, out=sel)
        if ev is not None:
            ev[1].record()
        gsa.build_layout(fixed, w.seq_len, 0, w.seq_len, bm, bn, out=tables)
        if ev is not None:
            ev[2].record()
        gsa.attn_prefill_unfolded(w.layout, tq, tk, tv, sel, tables, bm, bn, 0, scale, workspace=ws,
                                  out=(o, None))
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(2, args.steps // 2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    att_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    sl = sel.cpu().numpy()
    alg = 4.0 * w.d * unfolded_edges(w, sl) * (w.hq // w.hkv)
    S, c, g = w.n_sink, w.chunk_len, w.gists
    ncand = _counts(S, c, g, np.arange(w.seq_len))[0].astype(np.int64)
    sel_flops = 2.0 * w.d * float(ncand.sum()) * w.batch * w.hkv
    del tq, tk, tv, o, ws
    return {"workload": w.name, "ms_per_step": round(wall, 4), "select_ms": round(sel_ms, 4),
            "unfold_and_prefill_ms": round(att_ms, 4), "algorithmic_flops": alg,
            "tflops_algorithmic_step": round(alg / (wall * 1e-3) / 1e12, 2),
            "tflops_algorithmic_attention": round(alg / (att_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak_attention": round(alg / (att_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "selection_screen_flops": sel_flops,
            "selection_tflops": round(sel_flops / (sel_ms * 1e-3) / 1e12, 2),
            "kernels": "k_select_prefill; k_build_table; k_unfold + k_prefill_mfma (init from the unfold partial)"}


def blockmask_edges(flags: np.ndarray, block: int, w: int, n_bytes: int) -> tuple:
    """Visible (query, key) pairs of the gzip block masks of all sequences, in
    closed form per block pair, and the causal pairs of the same lengths."""
    nb = flags.shape[1]
    assert n_bytes == nb * block, "whole blocks only"
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    edges = 0
    for f in flags.astype(bool):
        linked = ((f[:, None] & f[None, :]) | (np.abs(i - j) <= w)) & (j < i)
        edges += int(linked.sum()) * block * block + nb * block * (block + 1) // 2
    causal = flags.shape[0] * n_bytes * (n_bytes + 1) // 2
    return edges, causal


def run_blockmask(wl, args, torch, gsa):
    """Gzip-guided block-mask prefill: host zlib flags (timed on their own),
    then one GPU step = gsa_build_block_mask + gsa_attn_prefill_blockmask."""
    from workloads import inputs
    dev = torch.device("cuda:0")
    x = inputs.mixed_bytes(wl.batch, wl.n_bytes, wl.block, seed=3)
    t0 = time.perf_counter()
    _, flags = gsa.gzip_block_flags(x, wl.block)
    host_ms = (time.perf_counter() - t0) * 1e3
    q, k, v = inputs.random_qkv(wl.batch, wl.n_bytes, wl.hq, wl.hkv, wl.d, seed=4, dtype="bf16")
    tq, tk, tv = (torch.from_numpy(a).to(dev).to(torch.bfloat16) for a in (q, k, v))
    tf = torch.from_numpy(flags).to(dev)
    bm, bn = gsa.prefill_tile(torch.bfloat16, wl.d)
    L = wl.n_bytes
    nqt, nkt = -(-L // bm), -(-L // bn)
    tables = (torch.empty((wl.batch, nqt, nkt), dtype=torch.int8, device=dev),
              torch.empty((wl.batch, nqt), dtype=torch.int32, device=dev),
              torch.empty((wl.batch, nqt, nkt), dtype=torch.int32, device=dev))
    o = torch.empty((wl.batch, L, wl.hq, wl.d), dtype=torch.bfloat16, device=dev)
    scale = 1 / math.sqrt(wl.d)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gsa.build_block_mask(tf, wl.block, wl.w, L, 0, L, bm, bn, out=tables)
        if ev is not None:
            ev[1].record()
        gsa.attn_prefill_blockmask(tq, tk, tv, tables, bm, bn, 0, scale, out=(o, None))
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(5, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    tab_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    att_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    edges, causal = blockmask_edges(flags, wl.block, wl.w, L)
    alg = 4.0 * wl.d * edges * wl.hq
    del tq, tk, tv, o
    return {"workload": wl.name, "ms_per_step": round(wall, 4), "table_ms": round(tab_ms, 4),
            "prefill_ms": round(att_ms, 4), "host_gzip_flags_ms": round(host_ms, 3),
            "edges": edges, "causal_edges": causal, "edge_fraction_of_causal": round(edges / causal, 4),
            "literal_block_fraction": round(float(flags.mean()), 4), "algorithmic_flops": alg,
            "tflops_algorithmic_prefill": round(alg / (att_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak_prefill": round(alg / (att_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": "k_block_mask_table; k_prefill_mfma<64> (one table per sequence)"}


def run_compact(w, args, torch, gsa, copies=2):
    """Fixed-layout decode over a compacted cache (sinks + gists + a window
    ring of raws): K/V of the whole sequence are drawn on the GPU (seeded),
    appended into `copies` independent compact caches, and one step = one
    gsa_compact_decode of the last position, timed by graph replay."""
    dev = torch.device("cuda:0")
    L, scale = w.seq_len, 1 / math.sqrt(w.d)
    gen = torch.Generator(device=dev)
    gen.manual_seed(21)
    cap = gsa.compact_gists(w.layout, L)
    slots = gsa.compact_slots(w.layout, cap)
    caches = []
    for _ in range(copies):
        kc = torch.empty((w.batch, w.hkv, slots, w.d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for p0 in range(0, L, 8192):   # appended in pieces, like a prefill writing its cache
            n = min(8192, L - p0)
            kn = torch.randn((w.batch, n, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
            vn = torch.randn((w.batch, n, w.hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
            gsa.compact_append(w.layout, kn, vn, p0, kc, vc, cap)
            del kn, vn
        caches.append((kc, vc))
    q = torch.randn((w.batch, w.hq, w.d), generator=gen, device=dev).to(torch.bfloat16)
    o = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(gsa.compact_decode_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L - 1),
                     dtype=torch.uint8, device=dev)

    def step(s):
        kc, vc = caches[s % copies]
        gsa.compact_decode(w.layout, q, kc, vc, L - 1, cap, scale, workspace=ws, out=(o, None))

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            for s in range(copies):
                step(s)
    torch.cuda.current_stream().wait_stream(st)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, max(args.steps, 20) // copies)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * copies)
    i = L - 1
    S, W1 = w.n_sink, max(w.window, 1)
    lo = max(0, i - W1 + 1)
    g_le, _ = _counts(w.n_sink, w.chunk_len, w.gists, np.array([i + 1]))
    _, r_hi = _counts(w.n_sink, w.chunk_len, w.gists, np.array([i + 1]))
    _, r_lo = _counts(w.n_sink, w.chunk_len, w.gists, np.array([lo]))
    rows = min(S, i + 1) + int(g_le[0]) + int(r_hi[0] - r_lo[0])
    nbytes = rows * w.batch * w.hkv * 2 * w.d * 2 + w.batch * w.hq * w.d * 2 * 2
    full_rows = L
    return {"workload": w.name, "ms_per_step": round(ms, 5), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "unique_bytes": int(nbytes), "visible_rows_per_group": rows,
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "cache_slots_per_group": slots, "full_cache_rows_per_group": full_rows,
            "kv_memory_saved": round(1 - slots / full_rows, 4),
            "kernels": "gsa_compact_decode (k_compact_decode)", "cache_copies": copies,
            "timing": "HIP graph of one step per cache copy, replayed; events on the replay stream"}


def profile_pass(torch, gsa, args):
    """A short pass for rocprofv3 counter runs: a 1 GiB device copy (to scale
    FETCH_SIZE / WRITE_SIZE), then two steps of one workload."""
    from workloads import configs, inputs
    dev = torch.device("cuda:0")
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = configs.BY_NAME[args.pass_workload]
    args.warmup, args.steps = 1, 1
    if args.pass_backward:
        q, k, v = inputs.prefill_inputs(w, seed=1)
        if w.top_k > 0:
            run_unfolded_backward(w, args, torch, gsa, q, k, v)
        else:
            run_backward(w, args, torch, gsa, q, k, v)
    elif w.kind == "blockmask":
        run_blockmask(w, args, torch, gsa)
    elif w.kind == "prefill":
        q, k, v = inputs.prefill_inputs(w, seed=1)
        if w.top_k > 0:
            run_unfolded(w, args, torch, gsa, q, k, v)
        else:
            run_prefill(w, args, torch, gsa, q, k, v)
    elif w.top_k == 0:
        run_compact(w, args, torch, gsa, copies=1)
    else:
        run_decode(w, args, torch, gsa, copies=1)
    torch.cuda.synchronize()
    print("profile pass done", flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-8b", action="store_true")
    ap.add_argument("--no-unfold", action="store_true")
    ap.add_argument("--no-blockmask", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6000)
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--pass-workload", default="llama3b_gqa24x8_ratio4_k0_prefill_32k")
    ap.add_argument("--pass-backward", action="store_true", help="profile pass: the backward of the workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(one process, one device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from workloads import configs, inputs
    w = configs.LLAMA3B_K0_PREFILL
    cpu = None
    if not args.profile_pass:
        q, k, v = inputs.prefill_inputs(w, seed=1)
        # host-only legs first: the oracle's worker processes fork before the GPU is touched
        log("inputs ready")
        if not args.no_cpu:
            cpu = cpu_baseline(w, q, k, v, args.cpu_rows)
            log(f"oracle baseline done: {cpu['sample']}")
            if not args.no_decode:
                cpu["decode"] = [cpu_baseline_decode(dw) for dw in (configs.SELECTIVE_DECODE, configs.HIER_DECODE)]
                log("oracle decode baselines done: " + ", ".join(f"{d['seconds']} s" for d in cpu["decode"]))

    import torch
    import gist_token_block_amd as gsa
    gsa.load_library()
    if args.profile_pass:
        profile_pass(torch, gsa, args)
        return

    p = run_prefill(w, args, torch, gsa, q, k, v)
    log(f"prefill {w.name}: {p['ms_per_step']:.3f} ms/step, kernel {p['kernel_ms']:.3f} ms")
    del q, k, v
    traffic = read_traffic()
    out = {
        "metric": METRIC, "value": p["tflops_visible_tile"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": p["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q,K,V ~ N(0,1) seeded, rounded to bf16",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.d, "positions": w.seq_len, "raw_tokens": 32768, "sinks": w.n_sink,
                   "chunk_len": w.chunk_len, "gists_per_chunk": w.gists, "window": w.window,
                   "top_k": w.top_k, "tile": p["tile"], "output": "bf16",
                   "step": "build_layout + attn_prefill"},
        "roofline": {"bound": "mfma", "achieved": p["tflops_algorithmic"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": p["frac_bf16_peak"], "traffic": traffic,
                     "kernel": "k_prefill_mfma<128, bf16 out>", "kernel_ms": p["kernel_ms"],
                     "algorithmic_flops": p["algorithmic_flops"],
                     "visible_tile_flops": p["visible_tile_flops"]},
        "source_sha": source_hash(),
    }
    if not args.no_8b:
        w8 = configs.LLAMA8B_K0_PREFILL
        q, k, v = inputs.prefill_inputs(w8, seed=2)
        p8 = run_prefill(w8, args, torch, gsa, q, k, v)
        del q, k, v
        log(f"prefill {w8.name}: {p8['ms_per_step']:.3f} ms/step, kernel {p8['kernel_ms']:.3f} ms")
        out["prefill"] = [p8]
    if not args.no_unfold:
        wu = configs.LLAMA3B_K16_PREFILL
        q, k, v = inputs.prefill_inputs(wu, seed=1)
        pu = run_unfolded(wu, args, torch, gsa, q, k, v)
        del q, k, v
        log(f"prefill {wu.name}: {pu['ms_per_step']:.3f} ms/step (select {pu['select_ms']:.3f} ms, "
            f"unfold + prefill {pu['unfold_and_prefill_ms']:.3f} ms)")
        out.setdefault("prefill", []).append(pu)
    if not args.no_backward:
        wbk = configs.LLAMA3B_K0_PREFILL
        q, k, v = inputs.prefill_inputs(wbk, seed=1)
        pbk = run_backward(wbk, args, torch, gsa, q, k, v)
        del q, k, v
        log(f"backward {wbk.name}: {pbk['ms_per_step']:.3f} ms/step, kernels {pbk['kernel_ms']:.3f} ms "
            f"({pbk['tflops_algorithmic']} TFLOP/s algorithmic)")
        out.setdefault("prefill", []).append(pbk)
        wuk = configs.LLAMA3B_K16_PREFILL
        q, k, v = inputs.prefill_inputs(wuk, seed=1)
        puk = run_unfolded_backward(wuk, args, torch, gsa, q, k, v)
        del q, k, v
        log(f"backward {wuk.name}: {puk['ms_per_step']:.3f} ms/step ({puk['tflops_algorithmic']} TFLOP/s "
            f"algorithmic)")
        out["prefill"].append(puk)
    if not args.no_blockmask:
        wb = configs.GZIP_BLOCKMASK_PREFILL
        pb = run_blockmask(wb, args, torch, gsa)
        log(f"prefill {wb.name}: {pb['ms_per_step']:.3f} ms/step (table {pb['table_ms']:.3f} ms, prefill "
            f"{pb['prefill_ms']:.3f} ms; host gzip flags {pb['host_gzip_flags_ms']:.1f} ms)")
        out.setdefault("prefill", []).append(pb)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if not args.no_decode:
        out["decode"] = []
        for dw in (configs.SELECTIVE_DECODE, configs.HIER_DECODE):
            torch.cuda.empty_cache()
            out["decode"].append(run_decode(dw, args, torch, gsa))
            log(f"decode {dw.name}: {out['decode'][-1]['ms_per_step'] * 1e3:.1f} us/step "
                f"(separate calls {out['decode'][-1]['separate_calls_ms_per_step'] * 1e3:.1f} us)")
        torch.cuda.empty_cache()
        out["decode"].append(run_compact(configs.COMPACT_DECODE, args, torch, gsa))
        log(f"decode {configs.COMPACT_DECODE.name}: {out['decode'][-1]['ms_per_step'] * 1e3:.1f} us/step")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
