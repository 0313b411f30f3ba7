"""Benchmark: ClusterKV sparse decode on one MI355X.

Workload (``llama8b-stack-32k-b8``): 32 Llama-3.1-8B-shaped layers, batch 8,
8 KV heads x 4 query heads, head_dim 128, 32768-token context per sequence
(16 sinks + 32752 clustered keys, 400 clusters per KV head, 10 Lloyd
rounds), recall budget 2048.  One *step* is one decode token for the whole
batch through all 32 layers: per layer ckv_append_select (the new token's
K/V row written and the recall, one launch) + ckv_sparse_decode.  Prefill clustering is timed separately (K-means keys/s).

Inputs are synthetic (seeded Gaussian-mixture keys on the GPU) and resident
in HBM before the timed region.  Each step is captured once as a HIP graph
(the per-step host counters differ, so every step has its own graph) and the
timed region replays them.  Prints one JSON line on stdout.
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

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "sparse-decode tokens/s & %HBM peak at 32k ctx, 2k budget; K-means keys/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(units: int, n_sink: int, c: int, r: int, group: int) -> int:
    """Algorithmic HBM bytes of one ckv_sparse_decode launch.

    Per unit: (n_sink + c + r) K and V rows of 256 B each, 4 B per recalled
    index, the bf16 query heads (2 G d) and the f32 output (4 G d).
    """
    d = 128
    return units * ((n_sink + c + r) * 2 * d * 2 + 4 * c + 2 * group * d + 4 * group * d)


def select_bytes(units: int, K: int, c: int, group: int, cut_rows: int) -> int:
    """Algorithmic HBM bytes of one ckv_select launch (cut_rows = mean cut-cluster size)."""
    d = 128
    return units * (4 * K * d + 8 * K + 4 + 2 * group * d + cut_rows * (2 * d + 4) + 4 * c)


# HBM bytes per ckv_sparse_decode launch on this workload, from two rocprofv3
# --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) scaled by what the
# same counters read for a plain 1 GiB device copy (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0).  Valid only for the kernel sources they were taken on:
# when the hash of those sources differs, traffic is reported as null.
TRAFFIC_SOURCES = ("decode.hip", "common.hpp")
TRAFFIC = {"sha256": "a727886e46567c8861703cf6bdc99d72e76965532d8f6a1b6363abe82ffb8081",
           "fetch_kib": 34308.39, "write_kib": 762.0}


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "semantic_cluster_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    if TRAFFIC["sha256"] is None or TRAFFIC["sha256"] != kernel_source_hash():
        return None
    return TRAFFIC["fetch_kib"] * 1024 * 2.0 + TRAFFIC["write_kib"] * 1024 * 1.0


def run_cpu_baseline(cfg, steps: int, seconds: float = 20.0) -> dict:
    """The oracle, untuned, on a bounded sample of the same workload (host cores)."""
    import numpy as np

    import synth
    from oracle import pipeline

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t_pre = t_dec = 0.0
    n_units = n_unit_steps = 0
    deadline = time.perf_counter() + seconds
    u = 0
    while time.perf_counter() < deadline and u < 64:
        kb, vb, cen = synth.make_unit_inputs(cfg.data_seed, u, cfg.n_tokens, cfg.components)
        init = synth.make_init_indices(cfg.init_seed, 1, cfg.m, cfg.n_clusters, unit_ids=[u])[0]
        t0 = time.perf_counter()
        st = pipeline.prefill_unit(kb, cfg.n_tokens, init, cfg.n_clusters, cfg.iters, v_bits=vb)
        t_pre += time.perf_counter() - t0
        n_units += 1
        for s in range(steps):
            q = synth.make_queries(cfg.query_seed, cen[None], cfg.group, step=s, unit_ids=[u])[0]
            t0 = time.perf_counter()
            sel = pipeline.select_unit(q, st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], cfg.budget)
            pipeline.decode_unit(q, kb, vb, st["k_clu_bits"], st["v_clu_bits"], sel["positions"], 16,
                                 cfg.n_tokens, cfg.n_tokens)
            t_dec += time.perf_counter() - t0
            n_unit_steps += 1
        u += 1
    units_total = cfg.layers * cfg.units
    step_s = t_dec / n_unit_steps * units_total
    return {
        "value": cfg.batch / step_s,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n_units} units x {steps} decode steps (select + decode, float64 NumPy) of the same "
                   f"workload, extrapolated to {units_total} units per step; prefill of the same "
                   f"{n_units} units timed for K-means keys/s"),
        "kmeans_keys_per_s": n_units * cfg.m / t_pre,
        "seconds": t_pre + t_dec,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (debug only)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 1 GiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by unit with no exchange, see DESIGN.md)", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "copies": 5}), flush=True)
        return 0

    import synth
    from synth import device as dgen
    from semantic_cluster_sparse_amd import ckv
    from semantic_cluster_sparse_amd.layer import Layer

    ckv.load_library()
    cfg = synth.CONFIGS["llama8b-stack-32k-b8"]
    n_layers = args.layers or cfg.layers
    W, K = args.warmup, args.steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cap = cfg.n_tokens + W + K + 1
    units, G, budget = cfg.units, cfg.group, cfg.budget
    stream = torch.cuda.current_stream()

    log(f"[bench] allocating {n_layers} layers of {units} units, capacity {cap}")
    layers = []
    qs = []
    for li in range(n_layers):
        L = Layer(batch=cfg.batch, n_kv_heads=cfg.n_kv_heads, group=G, n_clusters=cfg.n_clusters,
                  capacity=cap, max_budget=budget, incremental=False, device=dev)
        cen = dgen.fill_mixture(L.k_tok, L.v_tok, cfg.n_tokens, cfg.components, seed=10_000 + li)
        qs.append([dgen.queries(cen, G, seed=20_000 + 100 * li + s) for s in range(W + K)])
        del cen
        layers.append(L)
    torch.cuda.synchronize()
    log(f"[bench] generated inputs; {torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    # ---------------------------------------------------------------- prefill (timed separately)
    inits = [dgen.init_indices(units, cfg.m, cfg.n_clusters, seed=30_000 + li, device=dev)
             for li in range(n_layers)]
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for li, L in enumerate(layers):
        L.prefill(cfg.n_tokens, cfg.iters, inits[li])
    ev1.record(stream)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    prefill_ev_s = ev0.elapsed_time(ev1) / 1e3
    keys = n_layers * units * cfg.m
    log(f"[bench] prefill {prefill_s * 1e3:.1f} ms wall, {prefill_ev_s * 1e3:.1f} ms events; "
        f"{keys / prefill_ev_s / 1e6:.1f} M keys/s")
    del inits

    # ---------------------------------------------------------------- decode step buffers
    sel_pos = [torch.zeros((units, budget), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    cnt = [torch.zeros((units,), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    outs = [torch.zeros((units, G, 128), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    k_new = [dgen.rows(units, 128, 40_000 + s, dev) for s in range(W + K)]
    v_new = [dgen.rows(units, 128, 50_000 + s, dev) for s in range(W + K)]

    def step(s: int) -> None:
        for li, L in enumerate(layers):
            L.append_select(k_new[s], v_new[s], qs[li][s], budget, sel_pos[li], cnt[li])
            L.sparse_decode(qs[li][s], sel_pos[li], cnt[li], budget, outs[li])

    graphs = []
    if not args.no_graph:
        log("[bench] capturing one HIP graph per step")
        cs = torch.cuda.Stream()
        for s in range(W + K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                step(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(s: int) -> None:
        if graphs:
            graphs[s].replay()
        else:
            step(s)

    for s in range(W):
        run(s)
    torch.cuda.synchronize()
    log("[bench] warmup done; timing")
    t0 = time.perf_counter()
    for s in range(W, W + K):
        run(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / K * 1e3
    tokens_per_s = cfg.batch * K / dt
    log(f"[bench] {ms_per_step:.3f} ms/step, {tokens_per_s:.1f} tokens/s")

    # ---------------------------------------------------------------- kernel timing for the roofline
    # ckv_sparse_decode is one kernel per call.  The calls of all layers are
    # captured once more as a graph and replayed back to back between two
    # events on the stream they run on; the average is per launch.
    qlast = W + K - 1

    def decode_all() -> None:
        for li, L in enumerate(layers):
            L.sparse_decode(qs[li][qlast], sel_pos[li], cnt[li], budget, outs[li])

    if graphs:
        dg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dg, stream=cs):
            decode_all()
        launch_all = dg.replay
    else:
        launch_all = decode_all
    launch_all()
    torch.cuda.synchronize()
    reps = 5
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        launch_all()
    b.record(stream)
    torch.cuda.synchronize()
    dec_ms = a.elapsed_time(b) / (reps * n_layers)
    r_now = layers[0].n_total - layers[0].n_clustered
    dbytes = decode_bytes(units, 16, budget, r_now, G)
    achieved = dbytes / (dec_ms * 1e-3) / 1e9
    step_bytes = n_layers * (decode_bytes(units, 16, budget, (W + K) // 2, G)
                             + select_bytes(units, cfg.n_clusters, budget, G, 82) + units * 2 * 256)
    log(f"[bench] ckv_sparse_decode {dec_ms * 1e3:.1f} us/launch, {achieved:.0f} GB/s algorithmic")
    traffic = measured_traffic()

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": n_layers, "batch": cfg.batch, "kv_heads": cfg.n_kv_heads,
                   "group": G, "context": cfg.n_tokens, "clusters": cfg.n_clusters, "budget": budget,
                   "graphs": not args.no_graph},
        "roofline": {"bound": "hbm", "kernel": "ckv::sparse_decode_kernel<4>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "launch_us": dec_ms * 1e3, "bytes_per_launch": dbytes},
        "step_hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kmeans_keys_per_s": keys / prefill_ev_s,
        "prefill_ms": prefill_ev_s * 1e3,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host (bounded sample)")
        result["cpu_baseline"] = run_cpu_baseline(cfg, steps=3, seconds=args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
