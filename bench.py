#!/usr/bin/env python3
"""Routed history attention benchmark on one MI355X.

One step = one routed attention call of one layer at the chunk-48 shape
(40 heads, d = 128, bf16, 36 query blocks, 1692 history blocks, 60% of the
query blocks geometry-covered): block importance -> route selection -> sparse
attention, with q/k/v and the key-mean cache resident in HBM. The dense
attention of the same tensors is timed separately for the speedup.

Prints ONE JSON line on stdout (diagnostics go to stderr).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed attention latency/call (ms) + eff. TFLOP/s % MFMA peak at chunk-48 shape"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


KERNEL_SRC = os.path.join(ROOT, "geometry_routed_block_amd", "csrc", "velox_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_sparse_chunk48_traffic.json")


def measured_traffic():
    """HBM bytes per sparse-attention launch from the committed rocprofv3
    counter summary, or None when the kernel source changed since."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the attention kernel runs ~20% slower for its first ~10 launches after the
    # GPU idles (clock ramp): the default warmup covers that
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a "
                         "known-size reference for HBM byte counters)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the sparse-attention part of the oracle sample")
    ap.add_argument("--trace", type=str, default="",
                    help="comma-separated chunk numbers of the 48-chunk rollout (e.g. 1,2,4,8,16,32,48): "
                         "instead of the chunk-48 step, time the routed step and dense attention at "
                         "each chunk (one layer, 40 heads) and print the latency-vs-chunk curve")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the chunk-48 step, time the routed step and dense attention at the "
                         "chunk-48 shape with 0%%, 50%% and 100%% of the query blocks covered")
    ap.add_argument("--trace-layers", type=int, default=3,
                    help="layers (seeds 1000 + l) of the compact rollout trace folded into the default "
                         "JSON line (chunks 1, 2, 4, 7, 12, 24, 48); 0 skips it")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 0/50/100%% coverage sweep of the default JSON line")
    return ap.parse_args()


def run_trace(args):
    """Latency of the routed step (importance, routes, sparse attention) and of
    dense attention along the rollout: chunk c has 36 (c - 1) history blocks."""
    import numpy as np
    import torch

    import geometry_routed_block_amd as velox
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.sweep:
        cases = [(f"covered {int(f * 100)}%", (lambda f=f: synth.sweep(f))) for f in (0.0, 0.5, 1.0)]
    else:
        chunks = [int(c) for c in args.trace.split(",") if c.strip()]
        if not chunks or min(chunks) < 1 or max(chunks) > 48:
            raise SystemExit("--trace takes chunk numbers in 1..48")
        cases = [(c, (lambda c=c: synth.trace_chunk(c, layer=0))) for c in chunks]
    rows = []

    def timed(fn, warm, reps):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for c, make in cases:
        wl = make()
        q, k, v = synth.make_qkv(wl, device=dev)
        M = wl.M
        kbar = velox.block_mean(k[:, : M * 128]) if M > 0 else None
        g = torch.from_numpy(wl.g).to(dev)
        rho = torch.from_numpy(wl.rho).to(dev)
        coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(dev)
        L = velox.route_bound(wl.params, M)
        p = torch.zeros(wl.H, wl.N, M, dtype=torch.float32, device=dev)
        ids = torch.empty(wl.H, wl.N, max(L, 1), dtype=torch.int32, device=dev)
        lens = torch.empty(wl.H, wl.N, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        od = torch.empty_like(q)

        def step():
            if M > 0:
                velox.route_scores(q, kbar, M, out=p)
            velox.route_select(p, g, rho, coord, wl.params, L=max(L, 1), route_ids=ids, route_len=lens)
            velox.sparse_attn(q, k, v, ids, lens, M, out=o)

        routed = timed(step, args.warmup, args.steps)
        dense = timed(lambda: velox.dense_attn(q, k, v, M, out=od), 1, max(args.dense_steps, 1))
        tiles = int((lens.cpu().numpy() + wl.N).sum())
        rows.append({("covered" if args.sweep else "chunk"): c, "M": M, "routed_ms": round(routed, 4), "dense_ms": round(dense, 4),
                     "speedup": round(dense / routed, 3), "tiles_visited": tiles})
        log(f"{c}: M={M:4d}: routed {routed:.3f} ms, dense {dense:.3f} ms ({dense / routed:.2f}x), "
            f"{tiles} tiles")
        del q, k, v, kbar, o, od
        torch.cuda.empty_cache()
    if args.sweep:
        print(json.dumps({"metric": "routed step vs dense attention latency per call at the chunk-48 shape "
                                    "by covered fraction", "unit": "ms", "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": "chunk-48 coverage sweep (seeds 480-482)"},
                          "sweep": rows}), flush=True)
        return
    cross = next((r["chunk"] for r in rows if r["routed_ms"] < r["dense_ms"]), None)
    print(json.dumps({"metric": "routed step vs dense attention latency per call along the 48-chunk rollout",
                      "unit": "ms", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "48-chunk rollout trace: one layer (seed 1000), 40 heads, d 128, "
                                             "36 query blocks, 36 (c - 1) history blocks at chunk c"},
                      "first_chunk_routed_faster": cross, "trace": rows}), flush=True)


def _timed(fn, warm, reps):
    """Mean ms of `reps` back-to-back calls after `warm` untimed ones."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _routed_case(velox, q, k, v, kbar, wl, dev):
    """Buffers and the routed step (importance, routes, sparse attention) of a
    workload whose KV may be a prefix of a larger cache."""
    import numpy as np
    import torch
    M = wl.M
    g = torch.from_numpy(wl.g).to(dev)
    rho = torch.from_numpy(wl.rho).to(dev)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(dev)
    L = velox.route_bound(wl.params, M)
    p = torch.zeros(wl.H, wl.N, M, dtype=torch.float32, device=dev)
    ids = torch.empty(wl.H, wl.N, L, dtype=torch.int32, device=dev)
    lens = torch.empty(wl.H, wl.N, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    ws = velox.attn_workspace(q, L)

    def step():
        if M > 0:
            velox.route_scores(q, kbar, M, out=p)
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)
        velox.sparse_attn(q, k, v, ids, lens, M, out=o, workspace=ws)
    return step, lens, o


def compact_trace(layers, dev):
    """Routed step vs dense attention along the rollout, folded into the default
    line: chunks 1, 2, 4, 7, 12, 24, 48 of `layers` layers (seeds 1000 + l). Per
    layer one KV cache of 1728 blocks is drawn and chunk c uses its first
    36 c blocks (36 (c - 1) history blocks + the current chunk)."""
    import numpy as np
    import torch
    import geometry_routed_block_amd as velox
    import synth
    chunks = [1, 2, 4, 7, 12, 24, 48]
    routed = np.zeros((layers, len(chunks)))
    dense = np.zeros((layers, len(chunks)))
    tiles = np.zeros((layers, len(chunks)), np.int64)
    for ell in range(layers):
        full = synth.trace_chunk(48, ell)
        q, k, v = synth.make_qkv(full, device=dev)
        kbar = velox.block_mean(k[:, : full.M * 128])
        od = torch.empty_like(q)
        for ci, c in enumerate(chunks):
            wl = full if c == 48 else synth.trace_chunk(c, ell)
            T = (wl.M + wl.N) * 128
            kc, vc = k[:, :T], v[:, :T]
            step, lens, _ = _routed_case(velox, q, kc, vc, kbar, wl, dev)
            routed[ell, ci] = _timed(step, 3, 10)
            dense[ell, ci] = _timed(lambda: velox.dense_attn(q, kc, vc, wl.M, out=od), 1, 3)
            tiles[ell, ci] = int((lens.cpu().numpy() + wl.N).sum())
        log(f"trace layer {ell}: routed {np.round(routed[ell], 3).tolist()} dense {np.round(dense[ell], 3).tolist()}")
        del q, k, v, kbar, od
        torch.cuda.empty_cache()
    r_med, d_med = np.median(routed, axis=0), np.median(dense, axis=0)
    cross = next((c for c, r, d in zip(chunks, r_med, d_med) if r < d), None)
    return {"layers": layers, "seeds": [1000 + ell for ell in range(layers)], "chunks": chunks,
            "history_blocks": [36 * (c - 1) for c in chunks],
            "routed_ms": [round(float(x), 4) for x in r_med], "dense_ms": [round(float(x), 4) for x in d_med],
            "speedup": [round(float(d / r), 3) for r, d in zip(r_med, d_med)],
            "tiles_visited": [int(x) for x in np.median(tiles, axis=0)],
            "first_chunk_routed_faster": cross,
            "routed_ms_by_layer": [[round(float(x), 4) for x in row] for row in routed]}


def compact_sweep(dev):
    """Routed step vs dense at the chunk-48 shape with 0%, 50% and 100% of the
    query blocks covered (seeds 480-482)."""
    import torch
    import geometry_routed_block_amd as velox
    import synth
    out = {}
    for frac in (0.0, 0.5, 1.0):
        wl = synth.sweep(frac)
        q, k, v = synth.make_qkv(wl, device=dev)
        kbar = velox.block_mean(k[:, : wl.M * 128])
        step, lens, _ = _routed_case(velox, q, k, v, kbar, wl, dev)
        r = _timed(step, 3, 10)
        od = torch.empty_like(q)
        d = _timed(lambda: velox.dense_attn(q, k, v, wl.M, out=od), 1, 3)
        tiles = int((lens.cpu().numpy() + wl.N).sum())
        out[f"{int(frac * 100)}%"] = {"routed_ms": round(r, 4), "dense_ms": round(d, 4),
                                      "speedup": round(d / r, 3), "tiles_visited": tiles,
                                      "eff_tflops": round(4.0 * 128 ** 3 * tiles / (r * 1e-3) / 1e12, 1)}
        log(f"sweep covered {int(frac * 100)}%: routed {r:.3f} ms, dense {d:.3f} ms ({d / r:.2f}x)")
        del q, k, v, kbar, od
        torch.cuda.empty_cache()
    return out


def unique_tile_count(ids, lens, N, M):
    """Distinct (head, tile) pairs the sparse kernel reads (routed + current chunk)."""
    import numpy as np
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    total = 0
    for h in range(ids.shape[0]):
        seen = np.zeros(M, dtype=bool)
        for i in range(ids.shape[1]):
            seen[ids[h, i, : lens[h, i]]] = True
        total += int(seen.sum()) + N
    return total


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, q, k, v, p, ids, lens, seconds, max_rows=4096):
    """The oracle timed on a bounded sample, extrapolated to one whole call:
    importance and routes of one head, attention of rows drawn from every head
    (their tiles gathered to host memory outside the timed part), once with the
    BLAS pool as numpy sets it up and once on one thread."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        blas = 1
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = nproc
    rng = np.random.default_rng(0)

    qn0 = q[0:1].float().cpu().numpy()
    kn0 = k[0:1, : wl.M * 128].float().cpu().numpy()
    p_np = p[0].cpu().numpy()
    ids_np, lens_np = ids.cpu().numpy(), lens.cpu().numpy()
    t0 = time.perf_counter()
    oracle.importance(oracle.block_means(qn0), oracle.block_means(kn0), wl.scale)
    t_imp = time.perf_counter() - t0
    del kn0
    t0 = time.perf_counter()
    for i in range(wl.N):
        oracle.route_row(p_np[i], wl.g[i], wl.rho[i], wl.params, wl.M, wl.coords, i)
    t_route = time.perf_counter() - t0

    def gather(h, i):
        """Row (h, i) with its tiles (route, then the current chunk) packed."""
        import torch
        tiles = ids_np[h, i, : lens_np[h, i]].tolist() + list(range(wl.M, wl.M + wl.N))
        idx = torch.tensor(tiles, device=k.device)
        kt = k[h].view(-1, 128, k.shape[-1])[idx].reshape(1, -1, k.shape[-1])
        vt = v[h].view(-1, 128, v.shape[-1])[idx].reshape(1, -1, v.shape[-1])
        return (q[h:h + 1, i * 128:(i + 1) * 128].float().cpu().numpy(), kt.float().cpu().numpy(),
                vt.float().cpu().numpy(), len(tiles))

    def sample(budget, limit):
        done, spent = 0, 0.0
        while done < limit and (done < 8 or spent < budget):
            h, i = int(rng.integers(0, wl.H)), int(rng.integers(0, wl.N))
            qs, ks, vs, T = gather(h, i)
            t1 = time.perf_counter()
            oracle.attention_block(qs, ks, vs, wl.scale, 0, 0, range(T))
            spent += time.perf_counter() - t1
            done += 1
        return done, spent

    rows_n, t_attn = sample(seconds, max_rows)
    n_rows = wl.H * wl.N
    total_s = wl.H * t_imp + wl.H * t_route + n_rows / rows_n * t_attn
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1, t1 = sample(min(seconds, 8.0), 64)
        one = wl.H * t_imp + wl.H * t_route + n_rows / r1 * t1   # importance/routes barely use BLAS
    return {
        "value": round(total_s * 1e3, 1),
        "unit": "ms",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"importance of 1 head, routes of the {wl.N} rows of 1 head, sparse attention of "
                   f"{rows_n} (head, block) rows drawn with replacement from all {wl.H} heads; scaled to "
                   f"{wl.H} heads x {wl.N} rows (measured {t_imp + t_route + t_attn:.1f} s of CPU time)"),
        "nproc": int(nproc),
        "affinity_cpus": int(affinity),
        "cpu_model": _cpu_model(),
        "value_1core_ms": round(one * 1e3, 1) if one is not None else None,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; multi-GPU sharding is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    if args.trace or args.sweep:
        run_trace(args)
        return

    import numpy as np
    import torch

    import geometry_routed_block_amd as velox
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.chunk48()
    log(f"workload {wl.name}: H={wl.H} d={wl.d} N={wl.N} M={wl.M} {wl.dtype}")
    q, k, v = synth.make_qkv(wl, device=dev)
    kbar = velox.block_mean(k[:, : wl.M * 128])
    g = torch.from_numpy(wl.g).to(dev)
    rho = torch.from_numpy(wl.rho).to(dev)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(dev)
    L = velox.route_bound(wl.params, wl.M)
    p = torch.empty(wl.H, wl.N, wl.M, dtype=torch.float32, device=dev)
    ids = torch.empty(wl.H, wl.N, L, dtype=torch.int32, device=dev)
    lens = torch.empty(wl.H, wl.N, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    ws = velox.attn_workspace(q, L)
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src_buf = torch.ones(n, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del src_buf, dst_buf

    def step():
        velox.route_scores(q, kbar, wl.M, out=p)
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)
        velox.sparse_attn(q, k, v, ids, lens, wl.M, out=o, workspace=ws)

    # the rollout trace and the coverage sweep run first, so that the headline
    # warmup starts on a GPU that is already busy (after an idle period the
    # attention kernel runs slower for about its first ten launches)
    trace = compact_trace(args.trace_layers, dev) if args.trace_layers > 0 else None
    sweep = None if args.no_sweep else compact_sweep(dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    K = args.steps
    # the K timed steps, back to back: no event between the calls (a marker
    # costs the stream a few us of its own)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    # the per-call breakdown: the same K steps again, an event around each call
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for s in range(K):
        e = evs[s]
        e[0].record()
        velox.route_scores(q, kbar, wl.M, out=p)
        e[1].record()
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)
        e[2].record()
        velox.sparse_attn(q, k, v, ids, lens, wl.M, out=o, workspace=ws)
        e[3].record()
    torch.cuda.synchronize()
    t_scores = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_select = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_sparse = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    log(f"timed {K} steps: {ms_per_step:.3f} ms/step (scores {t_scores:.3f}, select {t_select:.3f}, "
        f"sparse {t_sparse:.3f})")

    # the same step with cold caches: 512 MiB read before each step (more than
    # the 8 x 4 MiB L2 and the 256 MiB MALL; a read leaves them holding clean
    # lines, where a write fill would leave dirty ones whose write-back the
    # step would pay), outside the timed events. Nothing synchronises inside
    # the loop: the host queues the step while the flush runs, so the events
    # time the GPU alone.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold_ev = []
    for s in range(K):
        flush.sum()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        velox.route_scores(q, kbar, wl.M, out=p)
        e[1].record()
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)
        e[2].record()
        velox.sparse_attn(q, k, v, ids, lens, wl.M, out=o, workspace=ws)
        e[3].record()
        cold_ev.append(e)
    torch.cuda.synchronize()
    cold = [[e[0].elapsed_time(e[3]), e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
            for e in cold_ev]
    cold = np.median(np.array(cold), axis=0)
    log(f"cold caches: {cold[0]:.3f} ms/step (scores {cold[1]:.3f}, select {cold[2]:.3f}, sparse {cold[3]:.3f})")

    # The router calls alone, without the event markers between them that the
    # breakdown above places around each (a marker costs the stream a few us,
    # which is large against these calls): R calls back to back between two
    # events after a GPU spin long enough for the host to queue them all (warm),
    # and R (flush, call) pairs less R flushes alone (cold).
    def gpu_per_call(body, R=20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(4_000_000)
        a.record()
        for _ in range(R):
            body()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / R

    def do_scores():
        velox.route_scores(q, kbar, wl.M, out=p)

    def do_select():
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)

    t_flush = min(gpu_per_call(lambda: flush.sum()) for _ in range(3))
    router_us = {}
    for name, fn in (("route_scores", do_scores), ("route_select", do_select)):
        warm = min(gpu_per_call(fn) for _ in range(3))
        both = min(gpu_per_call(lambda: (flush.sum(), fn())) for _ in range(3))
        router_us[name] = {"warm": round(warm * 1e3, 2), "cold": round((both - t_flush) * 1e3, 2)}
    del flush
    log(f"router calls alone (us): {router_us}")

    # the same step captured once in a HIP graph and replayed (no host launch
    # work per step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(max(args.warmup, 1)):
        graph.replay()
    torch.cuda.synchronize()
    gs_, ge_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gs_.record()
    for _ in range(K):
        graph.replay()
    ge_.record()
    torch.cuda.synchronize()
    graph_ms = gs_.elapsed_time(ge_) / K
    log(f"graph-replayed step: {graph_ms:.3f} ms")
    del graph

    # dense baseline on the same tensors
    od = torch.empty_like(q)
    velox.dense_attn(q, k, v, wl.M, out=od)
    torch.cuda.synchronize()
    ds, de = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ds.record()
    for _ in range(args.dense_steps):
        velox.dense_attn(q, k, v, wl.M, out=od)
    de.record()
    torch.cuda.synchronize()
    dense_ms = ds.elapsed_time(de) / args.dense_steps

    # geometry scorer on the same scene (once per chunk, not per layer: reported
    # beside the step, not in it)
    sc = wl.scene
    qo = torch.from_numpy(sc["obb_query"]).to(dev)
    ho = torch.from_numpy(sc["obb_hist"]).to(dev)
    qp = torch.from_numpy(sc["query_pts"]).to(dev)
    g_out = velox.slab_overlap(qo, ho, lattice=8)
    rho_out, mask_out = velox.slab_coverage(qp, ho)
    torch.cuda.synchronize()
    geo_ms = {}
    for name, fn in (("slab_overlap", lambda: velox.slab_overlap(qo, ho, lattice=8, out=g_out)),
                     ("slab_coverage", lambda: velox.slab_coverage(qp, ho, rho=rho_out,
                                                                   token_mask=mask_out))):
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(20):
            fn()
        ge.record()
        torch.cuda.synchronize()
        geo_ms[name] = round(gs.elapsed_time(ge) / 20, 4)
    # slab table of one decoded chunk (36 blocks) and the multiwarp of the
    # 60 cached first/last frames (4x token resolution) into chunk 48's camera
    import synth.geometry as sgeo
    hc, hd, hcam, hcob = sgeo.slab_inputs(n_chunks=1)
    hc, hd, hcam, hcob = (torch.from_numpy(x).to(dev) for x in (hc, hd, hcam, hcob))
    fr, fcams, fsize, fpin, tcam, tsize, tpin, qcells = sgeo.multiwarp_inputs()
    fr, fcams, tcam, qcells = (torch.from_numpy(x).to(dev) for x in (fr, fcams, tcam, qcells))
    ws = torch.empty(velox._lib.load().velox_multiwarp_workspace_size(fr.shape[0], *fsize, *tsize),
                     dtype=torch.uint8, device=dev)
    zq_b, _ = velox.multiwarp(fr, fcams, fsize, fpin, tcam, tsize, tpin, workspace=ws)
    for name, fn in (("slab_table_36_blocks", lambda: velox.slab_table(hc, hd, hcam, hcob, *tpin)),
                     ("multiwarp_60_frames", lambda: velox.multiwarp(fr, fcams, fsize, fpin, tcam, tsize, tpin,
                                                                     workspace=ws)),
                     ("token_points_4608", lambda: velox.token_points(qcells, zq_b, *tsize, tcam, *tpin))):
        fn()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(20):
            fn()
        ge.record()
        torch.cuda.synchronize()
        geo_ms[name] = round(gs.elapsed_time(ge) / 20, 4)
    log(f"geometry (ms): {geo_ms}")

    # comparison routers on the same tensors ([project] 03 · Results: matched
    # model-only route; [digest]: hard geometric top-K; head-shared routes)
    variants = {}
    o_var = torch.empty_like(q)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name, mode in (("model_only", 1), ("geometry_only", 2)):
        prm_v = wl.params.replace(mode=mode)
        ids_v = torch.empty_like(ids)
        lens_v = torch.empty_like(lens)

        def run_v():
            velox.route_select(p, g, rho, coord, prm_v, L=L, route_ids=ids_v, route_len=lens_v)
            velox.sparse_attn(q, k, v, ids_v, lens_v, wl.M, out=o_var)
        ms_v = timed(run_v)
        variants[name] = {"select_plus_attn_ms": round(ms_v, 4),
                          "tiles_visited": int((lens_v.cpu().numpy() + wl.N).sum())}
    logits_ws = torch.empty(wl.H, wl.N, wl.M, device=dev)
    p_sh = torch.empty(1, wl.N, wl.M, device=dev)
    ids_sh = torch.empty(1, wl.N, L, dtype=torch.int32, device=dev)
    lens_sh = torch.empty(1, wl.N, dtype=torch.int32, device=dev)

    def run_shared():
        velox.route_scores_shared(q, kbar, wl.M, logits=logits_ws, out=p_sh)
        velox.route_select(p_sh, g, rho, coord, wl.params, L=L, route_ids=ids_sh, route_len=lens_sh)
        velox.sparse_attn(q, k, v, ids_sh[0], lens_sh[0], wl.M, out=o_var)
    variants["head_shared"] = {"step_ms": round(timed(run_shared), 4),
                               "tiles_visited": int((lens_sh.cpu().numpy() + wl.N).sum()) * wl.H}
    log(f"variants: {variants}")

    # one GPU's share of the heads under head parallelism (5 of 40 heads, the
    # chunk-48 rows of those heads): 90 workgroups for 256 CUs unless each
    # row's tiles are split over several workgroups
    wl5 = synth.chunk48(heads=5)
    q5, k5, v5 = synth.make_qkv(wl5, device=dev)
    kbar5 = velox.block_mean(k5[:, : wl5.M * 128])
    p5 = velox.route_scores(q5, kbar5, wl5.M)
    ids5, lens5 = velox.route_select(p5, g, rho, coord, wl5.params, L=L)
    o5 = torch.empty_like(q5)
    share = {"heads": 5, "tiles_visited": int((lens5.cpu().numpy() + wl5.N).sum()), "sparse_ms": {},
             "dense_ms": {}}
    for n in (1, 2, 4, 8):
        ws5 = velox.split_workspace(q5, n) if n > 1 else None
        share["sparse_ms"][n] = round(timed(lambda: velox.sparse_attn(q5, k5, v5, ids5, lens5, wl5.M, out=o5,
                                                                      n_split=n, workspace=ws5)), 4)
        share["dense_ms"][n] = round(timed(lambda: velox.dense_attn(q5, k5, v5, wl5.M, out=o5, n_split=n,
                                                                    workspace=ws5)), 4)
    best = min(share["sparse_ms"], key=share["sparse_ms"].get)
    share["sparse_tflops_best"] = round(4.0 * 128 ** 2 * wl5.d * share["tiles_visited"]
                                        / (share["sparse_ms"][best] * 1e-3) / 1e12, 1)
    log(f"one GPU's share (5 heads): {share}")
    del q5, k5, v5, kbar5, p5, o5

    # KV append of one chunk in global order (once per chunk per layer, at
    # model QKV time: reported beside the step). 3 latent frames of 32 x 48
    # tokens = the 36 blocks of a chunk, written over the current chunk's rows
    # after every timing above is done.
    Tl, Hl, Wl = 3, 32, 48
    k_new = torch.randn(wl.H, Tl * Hl * Wl, wl.d, device=dev).to(k.dtype)
    v_new = torch.randn_like(k_new)
    kb_cache = torch.zeros(wl.H, wl.M + wl.N, wl.d, device=dev)
    cells = torch.from_numpy(velox.gilbert_curve(Wl, Hl)).to(dev)
    velox.kv_append(k_new, v_new, Tl, Hl, Wl, 47, cells, k, v, wl.M * 128, kbar=kb_cache)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(20):
        velox.kv_append(k_new, v_new, Tl, Hl, Wl, 47, cells, k, v, wl.M * 128, kbar=kb_cache)
    a1.record()
    torch.cuda.synchronize()
    append_ms = a0.elapsed_time(a1) / 20
    append_bytes = 4 * k_new.numel() * k_new.element_size() + wl.H * wl.N * wl.d * 4
    log(f"kv_append: {append_ms:.4f} ms, {append_bytes / append_ms / 1e6:.0f} GB/s")

    lens_np = lens.cpu().numpy()
    tiles = int((lens_np + wl.N).sum())
    blk = 128
    flop = 4.0 * blk * blk * wl.d * tiles
    flop_hist = 4.0 * blk * blk * wl.d * int(lens_np.sum())
    dense_flop = 4.0 * blk * blk * wl.d * wl.H * wl.N * (wl.M + wl.N)
    uniq = unique_tile_count(ids, lens, wl.N, wl.M)
    tile_bytes = 2 * blk * wl.d * 2                 # K + V of one tile, bf16
    qo_bytes = 2 * q.numel() * 2
    uniq_bytes = uniq * tile_bytes + qo_bytes
    eff_tflops = flop / (ms_per_step * 1e-3) / 1e12
    kern_tflops = flop / (t_sparse * 1e-3) / 1e12
    log(f"sparse kernel {kern_tflops:.1f} TFLOP/s ({100 * kern_tflops / PEAK_BF16_TFLOPS:.1f}% of "
        f"bf16 peak); dense {dense_ms:.3f} ms = {dense_flop / dense_ms / 1e9:.1f} TFLOP/s; "
        f"speedup {dense_ms / ms_per_step:.2f}x")

    result = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded q/k/v with per-block mean offsets; slab-OBB overlaps)",
        "config": {
            "workload": (f"chunk-48 routed attention: H={wl.H}, d={wl.d}, N={wl.N} query blocks, "
                         f"M={wl.M} history blocks, bf16, 60% covered, K_cov=80, K_unc=150, "
                         f"n_prev=36, 26-neighbour safeguards"),
            "global_batch": 1,
            "seq_len": (wl.M + wl.N) * blk,
        },
        "eff_tflops": round(eff_tflops, 1),
        "pct_mfma_peak": round(100 * eff_tflops / PEAK_BF16_TFLOPS, 2),
        "breakdown_ms": {"route_scores": round(t_scores, 4), "route_select": round(t_select, 4),
                         "sparse_attn": round(t_sparse, 4)},
        "cold_cache": {"ms_per_step": round(float(cold[0]), 4),
                       "breakdown_ms": {"route_scores": round(float(cold[1]), 4),
                                        "route_select": round(float(cold[2]), 4),
                                        "sparse_attn": round(float(cold[3]), 4)},
                       "note": "median over the timed steps, each after a 512 MiB read that evicts "
                               "L2 and MALL (leaving them clean)"},
        "router_us": dict(router_us, method="GPU time per call: 20 calls back to back (warm); 20 (512 MiB read, "
                                            "call) pairs less 20 reads (cold); no event between the calls"),
        "ms_per_step_graph_replay": round(graph_ms, 4),
        "dense_ms": round(dense_ms, 4),
        "dense_tflops": round(dense_flop / (dense_ms * 1e-3) / 1e12, 1),
        "speedup_vs_dense": round(dense_ms / ms_per_step, 3),
        "router_variants": variants,
        "head_share_split_rows": share,
        "geometry_ms": geo_ms,
        "kv_append": {"ms": round(append_ms, 4), "bytes": append_bytes,
                      "gbps": round(append_bytes / append_ms / 1e6, 1),
                      "frac_hbm": round(append_bytes / append_ms / 1e6 / PEAK_HBM_GBPS, 4)},
        "geometry_point_tests": {"slab_overlap": wl.N * wl.M * 512, "slab_coverage": wl.N * 128 * wl.M,
                                 "multiwarp_samples": int(fr.numel())},
        "tiles_visited": tiles,
        "history_flop_share": round(flop_hist / flop, 4),
        "rollout_trace": trace,
        "coverage_sweep": sweep,
        "order": ("rollout trace and coverage sweep, then the headline warmup and timed steps (no event between "
                  "the calls), then the same steps with an event around each call (breakdown_ms, roofline), the "
                  "cold-cache steps, graph replay, dense baseline and side measurements"),
        "roofline": {
            "bound": "mfma",
            "achieved": round(kern_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "traffic_note": None,
            "kernel": "velox::pp::attn_kernel<true> (routed, d 128, bf16)",
            "timing_note": ("achieved = tile-pair FLOP / mean duration of the velox_sparse_attn call from HIP "
                            "events on its stream; the call is the unit-plan launch plus the attention kernel"),
            "hbm_unique_bytes": uniq_bytes,
            "hbm_frac_unique": round(uniq_bytes / (t_sparse * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        },
        "cpu_baseline": None,
    }
    tr = measured_traffic()
    if tr is not None:
        result["roofline"]["traffic"] = int(tr["fetch_bytes"] + tr["write_bytes"])
        result["roofline"]["traffic_note"] = (
            f"rocprofv3 FETCH_SIZE x{tr['fetch_scale']} + WRITE_SIZE x{tr['write_scale']} per launch "
            f"(scales from a {tr['calib_mib']} MiB copy); fetch {tr['fetch_bytes'] / 1e9:.2f} GB, "
            f"write {tr['write_bytes'] / 1e9:.3f} GB")
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, p, ids, lens, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
