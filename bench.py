"""Benchmark of the gist-token sparse attention hot path on one MI355X.

Headline: block-sparse prefill of the Llama-3.2-3B attention shape at 32K raw
tokens (24 query / 8 KV heads, d=128, ratio 4: 1 gist after every 4 raw
tokens, 128 sinks, window 128, fixed layout k=0), bf16.  One step = build the
block-visibility table + run the prefill over it.  ``value`` is TFLOP/s on the
visible tiles (4 d x cells of the non-empty 128x64 tiles x batch x query heads,
per step time).  The same line carries the roofline of the prefill kernel, the
fp64 oracle timed on the host cores, and the two decode workloads (selective
unfolding, and two-level gist of gist) as GB/s of unique visible K/V bytes.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-decode] [--no-cpu]
    python bench.py --profile-pass   # short pass for rocprofv3 counter runs
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
KERNEL_SOURCES = ["gist_token_block_amd/csrc/prefill_mfma.hip", "gist_token_block_amd/csrc/gsa_internal.h"]


# ---------------------------------------------------------------- closed forms (accounting)
def _counts(S, c, g, x):
    """(gists, raws) at positions < x for an array x (single level)."""
    P = c + g
    y = np.maximum(0, x - S)
    f, r = y // P, y % P
    return g * f + np.maximum(0, r - c), c * f + np.minimum(r, c)


def fixed_layout_edges(w) -> int:
    """Visible (query, key) pairs per (batch, head) of a k=0 layout."""
    S, c, g, W1 = w.n_sink, w.chunk_len, w.gists, max(w.window, 1)
    i = np.arange(w.seq_len, dtype=np.int64)
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


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(launch_flops_unused=None):
    """HBM bytes per prefill launch from the committed counter summary, or None
    if the kernel changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sha") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
    S, c, g, W1 = w.n_sink, w.chunk_len, w.gists, max(w.window, 1)
    i = np.array(rows)
    lo = np.maximum(0, i - W1 + 1)
    gl, _ = _counts(S, c, g, lo)
    edges = int(((i - lo + 1) + np.minimum(S, lo) + gl).sum())
    flops = 4.0 * w.d * edges * w.batch * w.hq
    _POOL_ARGS.update(lay=lay, tm=tm, q=q, k=k, v=v, G=w.hq // w.hkv, pos=list(range(w.seq_len)),
                      scale=1 / math.sqrt(w.d), rows=rows)
    from threadpoolctl import threadpool_limits
    workers = min(w.hkv, os.cpu_count() or 1, 16)
    ctx = mp.get_context("fork")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ctx.Pool(workers) as pool:
            pool.map(_oracle_worker, range(w.hkv))
        dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(rows)} query rows spread over the 41088 positions x all {w.hq} heads "
                      f"(batch {w.batch}), fp64 numpy, {workers} processes x 1 BLAS thread, "
                      f"{dt:.1f} s wall"}


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
    return wall / args.steps * 1e3, kern_ms, table, (bm, bn)


def run_decode(w, args, torch, gsa, copies=4):
    """Decode step = score_select + attn_decode; caches rotate over `copies`
    independent buffers so the visible rows are not served from the 256 MB
    Infinity Cache of a previous step."""
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
    wsb = torch.zeros(gsa.decode_workspace_bytes(w.layout, w.batch, w.hq, w.hkv, w.d, L),
                      dtype=torch.uint8, device=dev)

    def step(s):
        kc, vc = caches[s % copies]
        gsa.score_select(w.layout, tq, kc, L, L - 1, scale, cache_layout=True, out=(sel, selg))
        gsa.attn_decode(w.layout, tq, kc, vc, sel, selg, scale, workspace=wsb, out=(o, None))

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    n = max(args.steps, 20)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(n):
        step(s)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / n
    # unique visible rows per (batch, KV head) from the selection actually made
    sl = sel.cpu().numpy()
    sg = selg.cpu().numpy() if selg is not None else None
    rows = 0
    S, c, g, W1 = w.n_sink, w.chunk_len, w.gists, max(w.window, 1)
    i = L - 1
    lo = max(0, i - W1 + 1)
    P = c + g
    for bb in range(w.batch):
        for h in range(w.hkv):
            if not w.hierarchical:
                n_g = g * ((lo - S) // P) + max(0, (lo - S) % P - c)
                starts = [S + m * P for m in sl[bb, h, 0] if m >= 0]
            else:
                G2, g2 = w.l2_chunks, w.l2_gists
                P2 = G2 * P + g2
                y = lo - S
                n_g = g2 * (y // P2) + max(0, y % P2 - G2 * P)
                for gr in sg[bb, h, 0]:
                    if gr >= 0:
                        n_g += sum(min(max(lo - (S + gr * P2 + j * P + c), 0), g) for j in range(G2))
                starts = [S + (m // G2) * P2 + (m % G2) * P for m in sl[bb, h, 0] if m >= 0]
            rows += min(S, lo) + n_g + (i - lo + 1) + sum(min(max(lo - s0, 0), c) for s0 in starts)
    nbytes = rows * 2 * w.d * 2 + w.batch * w.hq * w.d * 2 * 2 + sl.nbytes + (0 if sg is None else sg.nbytes)
    nbytes = int(nbytes)
    return {"workload": w.name, "ms_per_step": round(ms, 5),
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "unique_bytes": nbytes,
            "visible_rows_per_group": round(float(rows) / (w.batch * w.hkv), 2),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernels": "score_select + decode", "cache_copies": copies}


def profile_pass(torch, gsa, args):
    """A short pass for rocprofv3 counter runs: a 1 GiB device copy (to scale
    FETCH_SIZE / WRITE_SIZE), then two prefill steps of the headline workload."""
    from workloads import configs, inputs
    dev = torch.device("cuda:0")
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    w = configs.LLAMA3B_K0_PREFILL
    q, k, v = inputs.prefill_inputs(w, seed=1)
    args.warmup, args.steps = 1, 1
    run_prefill(w, args, torch, gsa, q, k, v)
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
    ap.add_argument("--cpu-rows", type=int, default=6000)
    ap.add_argument("--profile-pass", action="store_true")
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
        # host-only leg first: its worker processes fork before the GPU is touched
        log("inputs ready")
        if not args.no_cpu:
            cpu = cpu_baseline(w, q, k, v, args.cpu_rows)
            log(f"oracle baseline done: {cpu['sample']}")

    import torch
    import gist_token_block_amd as gsa
    gsa.load_library()
    if args.profile_pass:
        profile_pass(torch, gsa, args)
        return

    step_ms, kern_ms, table, (bm, bn) = run_prefill(w, args, torch, gsa, q, k, v)
    log(f"prefill done: {step_ms:.3f} ms/step, kernel {kern_ms:.3f} ms")
    edges = fixed_layout_edges(w)
    alg_flops = 4.0 * w.d * edges * w.batch * w.hq
    tile_flops = 4.0 * w.d * visible_tile_cells(w, table, bm, bn) * w.batch * w.hq
    value = tile_flops / (step_ms * 1e-3) / 1e12
    achieved = alg_flops / (kern_ms * 1e-3) / 1e12
    traffic = read_traffic()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q,K,V ~ N(0,1) seeded, rounded to bf16",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.d, "positions": w.seq_len, "raw_tokens": 32768, "sinks": w.n_sink,
                   "chunk_len": w.chunk_len, "gists_per_chunk": w.gists, "window": w.window,
                   "top_k": w.top_k, "tile": [bm, bn], "output": "bf16",
                   "step": "build_layout + attn_prefill"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "k_prefill_mfma<128, bf16 out>",
                     "kernel_ms": round(kern_ms, 4), "algorithmic_flops": alg_flops,
                     "visible_tile_flops": tile_flops},
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if not args.no_decode:
        del q, k, v
        out["decode"] = []
        for dw in (configs.SELECTIVE_DECODE, configs.HIER_DECODE):
            out["decode"].append(run_decode(dw, args, torch, gsa))
            log(f"decode {dw.name} done: {out['decode'][-1]['ms_per_step']:.4f} ms/step")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
