#!/usr/bin/env python3
"""Benchmark of CLEAR attention forward on one MI355X.

One step = one CLEAR attention layer (image-query tiles, text rows, and the
text-row merge) over Q, K, V already resident in HBM.  The workload is the
8192x8192 FLUX-1.dev shape: B 1, 24 heads, head_dim 128, a 512x512 token grid
plus 512 text tokens, bf16, seeded synthetic inputs (the generator of
dit_circular_local_amd.inputs).  The headline radius is r = 32; r = 8 is timed
the same way and reported alongside.

Metric: in-window attention TFLOP/s = 4 * d * (admitted pairs) * B * H / time,
counting only pairs the mask admits (image-window pairs, image->text pairs, and
the global text rows), as a fraction of the bf16 dense matrix-core peak.

Prints ONE JSON line on stdout (progress goes to stderr).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def admitted_pairs(n_text: int, gh: int, gw: int, r2: int, window: str = "circle") -> int:
    """Admitted (query, key) pairs of one head: for each window offset (dy, dx)
    with dy^2 + dx^2 <= r2, (gh - |dy|)(gw - |dx|) image queries have that key on
    the grid; image queries also admit the n_text text keys; text queries admit
    all N keys.  The square window (max(dy^2, dx^2) <= r2) factors into one sum
    per axis."""
    img = 0
    if r2 >= 0 and window == "square":
        w = math.isqrt(r2)
        img = (sum(gh - abs(d) for d in range(-w, w + 1) if abs(d) < gh)
               * sum(gw - abs(d) for d in range(-w, w + 1) if abs(d) < gw))
    elif r2 >= 0:
        w = math.isqrt(r2)
        for dy in range(-w, w + 1):
            if abs(dy) >= gh:
                continue
            half = math.isqrt(r2 - dy * dy)
            for dx in range(-half, half + 1):
                if abs(dx) < gw:
                    img += (gh - abs(dy)) * (gw - abs(dx))
    n = n_text + gh * gw
    return img + gh * gw * n_text + n_text * n


def computed_pairs(ca, n_text: int, gh: int, gw: int, r2: int, window: str = "circle") -> float:
    """Query-key products the kernels evaluate per head, tile waste included, in
    pair units (one pair = Q.K plus P.V work, 4d flops).  Per 32-query x 32-key
    chunk of a wavefront: Q.K and P.V run for text chunks and for the listed key
    tiles its sub-tile touches (masked pairs inside such a chunk included);
    untouched ones are skipped.  Text workgroups run every chunk of all N keys."""
    import numpy as np

    tm = ca.tile_map_build(gh, gw, r2, window=window)
    f = tm["flags"].astype(np.int64)
    nsub = (ca.TILE_H // ca.SUB_H) * (ca.TILE_W // ca.SUB_W)
    touched = sum(int(((f >> w) & 1).sum()) for w in range(nsub))
    ntiles = (-(-gh // ca.TILE_H)) * (-(-gw // ca.TILE_W))
    per_chunk = ca.CHUNK * 32
    text_chunks = -(-n_text // ca.CHUNK)
    dense = ntiles * nsub * text_chunks
    n = n_text + gh * gw
    text_rows = -(-n_text // 128) * 4 * (-(-n // ca.CHUNK))
    return (dense + touched + text_rows) * per_chunk


def load_profile(workload: str, radius: int):
    """Figures of the forward kernel from the committed rocprofv3 runs
    (profiles/traffic.json, written by dit_circular_local_amd.profiling), if they
    were taken on the current kernel sources and device flags (else None)."""
    from dit_circular_local_amd.build import kernel_source_hash

    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(f"{workload}_r{radius}")
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e


def time_layer(ca, torch, q, k, v, w, radius, steps, warmup, window="circle"):
    out = torch.empty_like(q)
    kw = {} if window == "circle" else {"window": window}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=radius, out=out, **kw)   # builds the tile map
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(warmup):
        ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=radius, out=out, **kw)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=radius, out=out, **kw)
        e.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ker = sorted(s.elapsed_time(e) for s, e in ev)
    return {
        "ms_per_step": wall_ms,
        "kernel_ms_mean": sum(ker) / len(ker),
        "kernel_ms_p10": ker[int(0.1 * (len(ker) - 1))],
        "kernel_ms_median": ker[len(ker) // 2],
        "kernel_ms_p90": ker[int(0.9 * (len(ker) - 1))],
        "first_call_ms": first_ms,
    }, out


def time_strips(ca, torch, q, k, v, w, radius, strips, steps, warmup):
    """The layer as `strips` horizontal strips (each one device's share in a
    patch-parallel run), run one after another on this GPU, then the text rows
    merged exactly and by the patch average (Eq. 7).  Returns per-strip and merge
    times (HIP events on the launch stream; the timed passes give strip 0 the text
    keys, as the exact merge needs) and the patch average's distance from the
    exact text rows."""
    B, H, N, d = q.shape
    out = torch.empty_like(q)
    po = torch.empty((strips, B * H, w.n_text, d), dtype=torch.float32, device=q.device)
    pml = torch.empty((strips, B * H, w.n_text, 2), dtype=torch.float32, device=q.device)
    rows = ca.strip_rows(w.grid_h, strips)
    stream = torch.cuda.current_stream()

    def one_pass(record=None):
        for s_, (y0, y1) in enumerate(rows):
            if record is not None:
                record[s_][0].record(stream)
            ca.fwd_strip(q, k, v, w.n_text, w.grid_h, w.grid_w, y0, y1, out, po[s_], pml[s_],
                         radius=radius, with_text_keys=(s_ == 0))
            if record is not None:
                record[s_][1].record(stream)
        if record is not None:
            record[-2][0].record(stream)
        ca.text_merge(po, pml, out, w.n_text, w.grid_h, w.grid_w, mode="exact")
        if record is not None:
            record[-2][1].record(stream)
            record[-1][0].record(stream)
        ca.text_merge(po, pml, out, w.n_text, w.grid_h, w.grid_w, mode="patch_average")
        if record is not None:
            record[-1][1].record(stream)

    for _ in range(warmup):
        one_pass()
    times = [[0.0] * (strips + 2) for _ in range(steps)]
    for it in range(steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(strips + 2)]
        one_pass(ev)
        torch.cuda.synchronize()
        times[it] = [a.elapsed_time(b) for a, b in ev]
    med = [sorted(t[i] for t in times)[steps // 2] for i in range(strips + 2)]
    halo_rows = math.isqrt(radius * radius)
    # how far the patch average (Eq. 7: every patch holds the text keys) lands from
    # the exact text rows
    ca.text_merge(po, pml, out, w.n_text, w.grid_h, w.grid_w, mode="exact")
    exact = out[:, :, :w.n_text].float().clone()
    for s_, (y0, y1) in enumerate(rows):
        ca.fwd_strip(q, k, v, w.n_text, w.grid_h, w.grid_w, y0, y1, out, po[s_], pml[s_],
                     radius=radius, with_text_keys=True)
    ca.text_merge(po, pml, out, w.n_text, w.grid_h, w.grid_w, mode="patch_average")
    diff = (out[:, :, :w.n_text].float() - exact).abs()
    torch.cuda.synchronize()
    return {
        "strips": strips,
        "rows_per_strip": w.grid_h // strips,
        "strip_ms_max": round(max(med[:strips]), 4),
        "strip_ms_min": round(min(med[:strips]), 4),
        "strips_ms_sum": round(sum(med[:strips]), 4),
        "merge_exact_ms": round(med[strips], 4),
        "merge_patch_average_ms": round(med[strips + 1], 4),
        "eq7_vs_exact_text_rows": {"max_abs": round(float(diff.max()), 5),
                                   "mean_abs": round(float(diff.mean()), 6),
                                   "exact_rms": round(float(exact.pow(2).mean().sqrt()), 5)},
        "halo_rows_per_side": halo_rows,
        "halo_bytes_per_neighbour": halo_rows * w.grid_w * H * d * 2 * q.element_size(),
    }


def time_backward(ca, torch, q, k, v, w, radius, steps, warmup):
    """The layer's gradients (clear_attn_bwd) for a seeded upstream gradient,
    given the forward's output and LSE (computed once, outside the timed
    region).  Returns ms per call from HIP events on the launch stream."""
    from dit_circular_local_amd.inputs import make_dout

    do = make_dout(w.B, w.H, w.n, w.d, w.dtype, seed=0, device=q.device)
    out, lse = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=radius, return_lse=True)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    for _ in range(warmup):
        ca.bwd(q, k, v, out, do, lse, w.n_text, w.grid_h, w.grid_w, radius=radius, grads=grads)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for s_, e_ in ev:
        s_.record(stream)
        ca.bwd(q, k, v, out, do, lse, w.n_text, w.grid_h, w.grid_w, radius=radius, grads=grads)
        e_.record(stream)
    torch.cuda.synchronize()
    ms = sorted(s_.elapsed_time(e_) for s_, e_ in ev)
    del do, out, lse, grads
    torch.cuda.empty_cache()
    return ms[len(ms) // 2], sum(ms) / len(ms)


def _oracle_units(w, index, workers, text_group=64):
    """Work units of one head for worker `index` of `workers`: groups of up to
    `text_group` text rows and whole rows of 8x8 image blocks, interleaved in
    proportion (any prefix holds about the same share of each), each worker
    starting at another place so that the pool covers different parts."""
    ntg = -(-w.n_text // text_group) if w.n_text > 0 else 0
    nby, nbx = -(-w.grid_h // 8), -(-w.grid_w // 8)
    units = []
    for t in range(ntg):
        g = (t + index * ntg // workers) % ntg
        rows = list(range(g * text_group, min(w.n_text, (g + 1) * text_group)))
        units.append(((t + 0.5) / ntg, "text", rows))
    for b in range(nby):
        by = (b + index * nby // workers) % nby
        units.append(((b + 0.5) / nby, "blocks", [(by, bx) for bx in range(nbx)]))
    units.sort(key=lambda u: u[0])
    return [(kind, payload) for _, kind, payload in units]


def _oracle_worker(args):
    """One worker of the CPU baseline.  For each job (workload, radius, time
    budget) in turn: regenerate head `index` mod H of the workload from the
    seeded generator, widen it to float64, wait for the other workers, then run
    the fp64 oracle over the head's work units until the head is done or the
    budget is spent.  Returns per job (admitted pairs, text rows, block rows,
    seconds, units done, units), and the BLAS threads of the worker."""
    (jobs, seed, index, workers, barrier) = args
    from dit_circular_local_amd.inputs import WORKLOADS, make_head
    from oracle import attention_head, in_window_pairs

    # one BLAS thread per worker; the limit applies to the libraries already
    # loaded, so it comes after the imports that load numpy's BLAS (the pool's
    # environment sets the thread counts to 1 as well)
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(1)
        blas_threads = max((i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"),
                           default=None)
    except Exception:
        pass
    import torch
    torch.set_num_threads(1)

    out = []
    for wname, radius, budget_s in jobs:
        w = WORKLOADS[wname]
        head = index % w.H
        # widened to float64 here, outside the timed region (the oracle would
        # otherwise widen the whole head again on every call)
        qh, kh, vh = (make_head(w.n, w.d, t, 0, head, seed, w.dtype, w.rms_norm, w.scale).double().numpy()
                      for t in ("q", "k", "v"))
        r2 = radius * radius
        units = _oracle_units(w, index, workers)
        text_rows, blocks, done = [], [], 0
        barrier.wait()
        t0 = time.perf_counter()
        for kind, payload in units:
            if done and time.perf_counter() - t0 >= budget_s:
                break
            if kind == "text":
                attention_head(qh, kh, vh, w.n_text, w.grid_h, w.grid_w, r2, text_rows=payload, blocks=[])
                text_rows += payload
            else:
                attention_head(qh, kh, vh, w.n_text, w.grid_h, w.grid_w, r2, text_rows=[], blocks=payload)
                blocks += payload
            done += 1
        secs = time.perf_counter() - t0
        pairs = in_window_pairs(w.n_text, w.grid_h, w.grid_w, r2, text_rows=text_rows, blocks=blocks)
        out.append((pairs, len(text_rows), len(blocks) // max(1, -(-w.grid_w // 8)), secs, done, len(units)))
        del qh, kh, vh
    return out, blas_threads


def cpu_oracle_runs(jobs, seed=0):
    """The fp64 oracle, untuned, over a process pool on the host's cores: one
    worker per core (at most 16), one BLAS thread each, every worker on its own
    head.  `jobs` is a list of (workload, radius, seconds): the workers take the
    jobs in order, all at once (a barrier starts each job), each running whole
    heads where the budget allows and a proportional sample of text-row groups
    and image block rows where it does not.  Returns one record per job, in the
    metric's unit: 4 d x admitted pairs covered / the slowest worker's seconds."""
    import multiprocessing as mp

    from dit_circular_local_amd.inputs import WORKLOADS

    ncpu = os.cpu_count() or 1
    workers = max(1, min(ncpu, 16))
    ctx = mp.get_context("spawn")  # the parent holds a GPU context: never fork it
    # the workers inherit the environment when they start: one BLAS / OpenMP
    # thread each (hosts may set these to the core count, and 16 workers x 16
    # spinning BLAS threads on 16 cores starve every worker)
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in keys}
    os.environ.update({k: "1" for k in keys})
    try:
        with ctx.Manager() as mgr:
            barrier = mgr.Barrier(workers)
            args = [(list(jobs), seed, i, workers, barrier) for i in range(workers)]
            with ctx.Pool(workers) as pool:
                res = pool.map(_oracle_worker, args)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    blas = max((b for _, b in res if b is not None), default=None)
    records = []
    for j, (wname, radius, budget_s) in enumerate(jobs):
        w = WORKLOADS[wname]
        per = [r[0][j] for r in res]
        pairs = sum(x[0] for x in per)
        secs = max(x[3] for x in per)
        tflops = 4.0 * w.d * pairs / secs / 1e12 if secs > 0 else None
        whole = all(x[4] == x[5] for x in per)
        heads = sorted(set(i % w.H for i in range(workers)))
        layer_flops = 4.0 * w.d * admitted_pairs(w.n_text, w.grid_h, w.grid_w, radius * radius) * w.B * w.H
        nby = -(-w.grid_h // 8)
        records.append({
            "value": tflops,
            "unit": "TFLOP/s",
            "cores": workers,
            "kind": "oracle",
            "sample": (f"{workers} worker processes on heads {heads}: "
                       + ("each its whole head" if whole else
                          f"each a proportional share of its head's groups of 64 text rows and rows of 8x8 image "
                          f"blocks for ~{budget_s:g} s ({sum(x[1] for x in per)} text rows and "
                          f"{sum(x[2] for x in per)} block rows over all workers; a head has {w.n_text} text rows "
                          f"and {nby} block rows)")
                       + f", r={radius}; {pairs} admitted pairs in {secs:.2f} s; fp64 numpy"),
            "seconds": secs,
            "whole_heads": whole,
            "os_cpu_count": ncpu,
            "worker_processes": workers,
            "blas_threads_per_worker": blas,
            "radius": radius,
            "full_layer_seconds_extrapolated": layer_flops / (tflops * 1e12) if tflops else None,
        })
    return records


def cpu_baseline(w, radius, budget_s, seed=0):
    """The CPU baseline of one workload at one radius (see cpu_oracle_runs)."""
    return cpu_oracle_runs([(w.name, radius, budget_s)], seed)[0]


def time_configs(ca, torch, steps=5, warmup=2):
    """Every workload configuration the parity tests cover (tiny fp32, and the
    1024^2 .. 8192^2 FLUX shapes at each of their radii): ms per layer (median
    of `steps` calls, HIP events) and in-window TFLOP/s."""
    from dit_circular_local_amd.inputs import WORKLOADS, workload_qkv

    out = {}
    for name in ("tiny", "flux1k", "flux2k", "flux4k", "flux8k"):
        w = WORKLOADS[name]
        q, k, v = workload_qkv(w, seed=0, device="cuda")
        for r in w.radii:
            t, _ = time_layer(ca, torch, q, k, v, w, r, steps, warmup)
            flops = 4.0 * w.d * admitted_pairs(w.n_text, w.grid_h, w.grid_w, r * r) * w.B * w.H
            out[f"{name}_r{r}"] = {
                "ms_per_layer": round(t["kernel_ms_median"], 4),
                "in_window_tflops": round(flops / (t["kernel_ms_median"] * 1e-3) / 1e12, 3),
                "pct_bf16_peak": round(100.0 * flops / (t["kernel_ms_median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)
                if w.dtype == "bf16" else None,
                "dtype": w.dtype,
            }
            log(f"config {name} r={r}: {t['kernel_ms_median']:.4f} ms, {out[f'{name}_r{r}']['in_window_tflops']} TFLOP/s")
        del q, k, v
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux8k")
    ap.add_argument("--radius", type=int, default=32)
    ap.add_argument("--also-radius", type=int, default=8, help="second radius timed alongside (-1: none)")
    ap.add_argument("--square-radius", type=int, default=32,
                    help="also time the square-window variant at this radius (-1: none)")
    ap.add_argument("--strips", type=int, default=8,
                    help="also time the layer as this many horizontal strips plus text merges (0: none)")
    ap.add_argument("--backward-radii", default="32,8",
                    help="also time the backward (clear_attn_bwd) at these radii ('' : none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle work per worker and radius for the CPU baseline")
    ap.add_argument("--cpu-config-seconds", type=float, default=4.0,
                    help="oracle work per worker for each other configuration (at most a whole head)")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the other workload configurations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times) and exit: "
                         "the reference for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "the CLEAR attention layer here runs on a single MI355X", file=sys.stderr)
        sys.exit(2)

    import torch

    import dit_circular_local_amd as ca
    from dit_circular_local_amd.inputs import WORKLOADS, workload_qkv

    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_probe_mib} MiB x3")
        return
    w = WORKLOADS[args.workload]
    log(f"generating {w.name} inputs (seeded)...")
    t0 = time.perf_counter()
    q, k, v = workload_qkv(w, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    results = {}
    radii = [args.radius] + ([args.also_radius] if args.also_radius >= 0 and args.also_radius != args.radius else [])
    for r in radii:
        t, _ = time_layer(ca, torch, q, k, v, w, r, args.steps, args.warmup)
        pairs = admitted_pairs(w.n_text, w.grid_h, w.grid_w, r * r)
        flops = 4.0 * w.d * pairs * w.B * w.H
        cpairs = computed_pairs(ca, w.n_text, w.grid_h, w.grid_w, r * r)
        t["in_window_tflops"] = flops / (t["ms_per_step"] * 1e-3) / 1e12
        t["pct_bf16_peak"] = 100.0 * t["in_window_tflops"] / PEAK_BF16_TFLOPS
        t["computed_tflops"] = 4.0 * w.d * cpairs * w.B * w.H / (t["ms_per_step"] * 1e-3) / 1e12
        t["flops_per_layer"] = flops
        t["admitted_pairs_per_head"] = pairs
        t["computed_pairs_per_head"] = cpairs
        results[r] = t
        log(f"r={r}: {t['ms_per_step']:.3f} ms/layer, {t['in_window_tflops']:.1f} TFLOP/s in-window "
            f"({t['pct_bf16_peak']:.1f}% of bf16 peak), kernel {t['kernel_ms_mean']:.3f} ms")

    square = None
    if args.square_radius >= 0:
        r = args.square_radius
        t, _ = time_layer(ca, torch, q, k, v, w, r, args.steps, args.warmup, window="square")
        pairs = admitted_pairs(w.n_text, w.grid_h, w.grid_w, r * r, "square")
        flops = 4.0 * w.d * pairs * w.B * w.H
        cpairs = computed_pairs(ca, w.n_text, w.grid_h, w.grid_w, r * r, "square")
        square = {
            "radius": r,
            "ms_per_layer": round(t["ms_per_step"], 4),
            "in_window_tflops": round(flops / (t["ms_per_step"] * 1e-3) / 1e12, 3),
            "pct_bf16_peak": round(100.0 * flops / (t["ms_per_step"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "computed_tflops": round(4.0 * w.d * cpairs * w.B * w.H / (t["ms_per_step"] * 1e-3) / 1e12, 3),
            "admitted_pairs_per_head": pairs,
        }
        log(f"square window r={r}: {t['ms_per_step']:.3f} ms/layer, {square['in_window_tflops']:.1f} TFLOP/s in-window")

    main_r = args.radius
    m = results[main_r]
    achieved = m["flops_per_layer"] / (m["kernel_ms_mean"] * 1e-3) / 1e12
    prof = load_profile(w.name, main_r)
    traffic = prof.get("hbm_bytes_per_launch") if prof else None
    line = {
        "metric": "in-window attention TFLOP/s (CLEAR forward, 8192x8192, r=32; ms/layer and r=8 alongside)",
        "value": round(m["in_window_tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"CLEAR attention forward {w.name}: B{w.B} H{w.H} d{w.d}, "
                        f"{w.grid_h}x{w.grid_w} grid + {w.n_text} text tokens, r={main_r}",
            "B": w.B, "H": w.H, "d": w.d, "n_text": w.n_text, "grid_h": w.grid_h, "grid_w": w.grid_w,
            "radius": main_r,
        },
        "pct_bf16_peak": round(m["pct_bf16_peak"], 2),
        "ms_per_layer": {"median": round(m["kernel_ms_median"], 4), "p10": round(m["kernel_ms_p10"], 4),
                         "p90": round(m["kernel_ms_p90"], 4)},
        "computed_tflops": round(m["computed_tflops"], 3),
        "tilemap_first_call_ms": round(m["first_call_ms"], 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "clear_attn_fwd_kernel<Bf16G> + clear_text_merge_kernel (HIP events around each call)",
            # from the committed counter runs of these sources (null when they changed since):
            # matrix-core busy share of SIMD cycles, and the fabric bytes above per this run's
            # mean launch time
            "mfma_util": round(prof["mfma_busy"], 4) if prof and prof.get("mfma_busy") else None,
            "hbm_gbps": round(traffic / (m["kernel_ms_mean"] * 1e-3) / 1e9, 1) if traffic else None,
            "profile_kernel_ms": round(prof["kernel_ms"], 4) if prof and prof.get("kernel_ms") else None,
        },
    }
    # the pages' figures, context only (another machine, and end-to-end numbers
    # that include the rest of the DiT): 99.5 % attention-compute reduction and
    # 6.3x generation speed-up at 8192^2 (293.5 s vs 1842.5 s per 50 steps, r = 8;
    # atlas.scime.ai summary of CLEAR, "Key results"), beside the reduction this
    # layer's own admitted-pair counts give
    dense_pairs = w.n * w.n
    line["pages_context"] = {
        "attention_compute_reduction_pages": 0.995,
        "end_to_end_speedup_pages": 6.3,
        "seconds_per_50_steps_8192_pages": {"clear_r8": 293.5, "flux_1_dev": 1842.5},
        "hardware_pages": "not stated on the pages",
        "attention_compute_reduction_here": {
            f"r{r}": round(1.0 - admitted_pairs(w.n_text, w.grid_h, w.grid_w, r * r) / dense_pairs, 5)
            for r in radii},
    }
    for r in radii[1:]:
        t = results[r]
        line[f"r{r}"] = {
            "ms_per_layer": round(t["ms_per_step"], 4),
            "in_window_tflops": round(t["in_window_tflops"], 3),
            "pct_bf16_peak": round(t["pct_bf16_peak"], 2),
            "computed_tflops": round(t["computed_tflops"], 3),
        }
    if square is not None:
        line[f"square_r{square['radius']}"] = square
    if args.strips > 0:
        st = time_strips(ca, torch, q, k, v, w, main_r, args.strips, min(args.steps, 10), 2)
        line[f"strips{args.strips}"] = st
        log(f"{args.strips} strips: max {st['strip_ms_max']:.3f} ms per strip, sum {st['strips_ms_sum']:.3f} ms, "
            f"merges {st['merge_exact_ms']:.3f} / {st['merge_patch_average_ms']:.3f} ms")
    for r in [int(x) for x in args.backward_radii.split(",") if x.strip()]:
        med, mean = time_backward(ca, torch, q, k, v, w, r, min(args.steps, 10), 2)
        # the backward's algorithmic work: 5 products of 2d flops per admitted
        # pair (S recomputed, dP, dV, dK, dQ) = 2.5x the forward's 4d
        bflops = 2.5 * 4.0 * w.d * admitted_pairs(w.n_text, w.grid_h, w.grid_w, r * r) * w.B * w.H
        line[f"backward_r{r}"] = {
            "ms_per_layer": round(med, 4),
            "ms_mean": round(mean, 4),
            "in_window_tflops": round(bflops / (med * 1e-3) / 1e12, 3),
            "pct_bf16_peak": round(100.0 * bflops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "flops_per_layer": bflops,
        }
        log(f"backward r={r}: {med:.3f} ms/layer, {line[f'backward_r{r}']['in_window_tflops']:.1f} TFLOP/s in-window")
    if not args.no_configs:
        line["configs"] = time_configs(ca, torch)
    if not args.no_cpu_baseline:
        del q, k, v
        torch.cuda.empty_cache()
        from dit_circular_local_amd.inputs import WORKLOADS as _W

        jobs = [(w.name, r, args.cpu_seconds) for r in radii]
        if "configs" in line:
            jobs += [(name, r, args.cpu_config_seconds) for name in ("tiny", "flux1k", "flux2k", "flux4k", "flux8k")
                     for r in _W[name].radii]
        log(f"timing the CPU oracle: {len(jobs)} runs ({args.cpu_seconds:.0f} s per worker at the headline "
            f"radii, {args.cpu_config_seconds:.0f} s per configuration or a whole head)...")
        try:
            recs = cpu_oracle_runs(jobs)
        except Exception as e:  # the GPU figures stand without the CPU baseline
            log(f"CPU oracle runs failed: {e!r}")
            recs = [{"value": None, "unit": "TFLOP/s", "kind": "oracle", "error": repr(e)} for _ in jobs]
        for (name, r, _), cb in zip(jobs[:len(radii)], recs):
            line["cpu_baseline" if r == main_r else f"cpu_baseline_r{r}"] = cb
            if cb["value"] is not None:
                log(f"CPU oracle r={r}: {cb['value']:.4f} TFLOP/s on {cb['worker_processes']} processes")
        for (name, r, _), cb in zip(jobs[len(radii):], recs[len(radii):]):
            line["configs"][f"{name}_r{r}"]["cpu_oracle"] = {
                k: cb[k] for k in ("value", "unit", "seconds", "whole_heads", "worker_processes", "sample", "error")
                if k in cb}
            ratio = line["configs"][f"{name}_r{r}"]["in_window_tflops"] / cb["value"] if cb["value"] else None
            line["configs"][f"{name}_r{r}"]["gpu_over_cpu_oracle"] = round(ratio, 1) if ratio else None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
