"""Benchmark: ClusterKV sparse decode on one MI355X.

Default workload (``llama8b-stack-32k-b8``): 32 Llama-3.1-8B-shaped layers,
batch 8, 8 KV heads x 4 query heads, head_dim 128, 32768-token context per
sequence (16 sinks + 32752 clustered keys, 400 clusters per KV head, 10 Lloyd
rounds), recall budget 2048.  One *step* is one decode token for the whole
batch through all layers: per layer one ckv_append_select_decode launch (the
new token's K/V row written, the recall and the sparse attention).  With
``--separate`` the step runs the two-launch form instead (ckv_append_select,
then ckv_sparse_decode).  Prefill clustering is timed separately (K-means
keys/s).

``--workload glm4-stack-32k-b16``: 40 GLM4-9B-shaped layers (2 KV heads x 16
query heads), batch 16, 32468 clustered + 300 recent tokens, 410 clusters,
budget 2048, 50 steps; a step that finds 320 recent tokens first calls
ckv_cluster_incremental on every layer, so the timed steps include one
re-clustering.  Reports steady-state tokens/s with the re-clustering spread
over its 320 steps.  With ``--async-recluster`` the re-clustering runs as
ckv_cluster_incremental_async on a second stream beside the decode steps and
is committed ``--async-lag`` steps later (the steps in between still see the
old clusters plus a growing recent window).

``--workload llama8b-incremental-b16``: one Llama layer at batch 16 (128
units), 32768 clustered tokens, then 320 new keys per KV head (10% from 8
new mixture components): times ckv_cluster_incremental, then a budget-1024
ckv_select and ckv_sparse_decode on batch-16 queries.  Reports the
incremental latency.  With ``--split-reserve R`` the prefill holds R cluster
slots per unit empty and ckv_cluster_split is timed after the incremental
call (threshold: the median drift).

``--per-head-recall`` switches the stack workloads to the other grouped-query
reading: ckv_append + ckv_select_decode_per_head (with ``--separate``:
ckv_append + ckv_select_per_head + ckv_sparse_decode_per_head), one recalled
set per query head.

``roofline`` prices the kernel the step spends its time in: the fused recall +
decode launch on its algorithmic bytes (the decode's rows, positions, queries
and output plus the recall's centroids, offsets and unkept cut-cluster keys),
or ckv_sparse_decode on the decode's bytes in the two-launch form.

The stack workloads also time a dense-decode baseline on the same harness
(``full_attention``): budget >= m, so recall takes every cluster and the
decode kernel attends to all cached tokens; and the assignment step alone
(``assign_roofline``: ckv_assign over every layer after the prefill, against
the bf16 MFMA peak).

``--workload single-head-2k`` and ``--workload llama8b-layer-32k``: one
layer (1 unit with one query head, K = 24, budget 256; or 8 KV heads x 4
query heads, K = 400, budget 1024) through the same prefill and 200 fused
decode steps; their ``cpu_baseline`` times the oracle on every unit.

Every line reports the measured 1 GiB device-copy rate beside the HBM peak
(``roofline.copy_gbs``, ``roofline.frac_of_copy``).

Inputs are synthetic (seeded Gaussian-mixture keys on the GPU) and resident
in HBM before the timed region.  Decode steps are captured once each as a HIP
graph (the per-step host counters differ, so every step has its own graph)
and the timed region replays them.  Prints one JSON line on stdout.
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
MFMA_BF16_PEAK_TFS = 2500.0   # MI355X dense bf16 MFMA, 2.5 PFLOP/s
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


# Mean number of a cut cluster's tokens that recall scores but does not keep
# (about half of an 82-token cluster at 400 clusters over 32752 keys).
CUT_UNKEPT_ROWS = 41


def fused_bytes(units: int, n_sink: int, c: int, r: int, group: int, K: int) -> int:
    """Algorithmic HBM bytes of one ckv_select_decode launch.

    Per unit: the attended K and V rows (n_sink + c + r rows of 256 B each),
    the recalled positions written (4 c), the query heads (2 G d) and the f32
    output (4 G d) -- exactly the decode's bytes -- plus what the recall reads
    on top: the scoring centroids (4 K d), the cluster offsets (4 (K + 1)), the
    recalled count written (4) and the keys of the cut cluster's tokens that
    are scored but not kept (CUT_UNKEPT_ROWS rows of 2 d).  The centroids are
    counted once although every chunk of a set reads them (they come from L2
    after the first).
    """
    d = 128
    return (decode_bytes(units, n_sink, c, r, group)
            + units * (4 * K * d + 4 * (K + 1) + 4 + CUT_UNKEPT_ROWS * 2 * d))


# HBM bytes per launch of the priced kernel on the default workload, from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) scaled by
# what the same counters read for a plain 1 GiB device copy (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0).  Valid only for the kernel sources they were taken on:
# when the hash of those sources differs, traffic is reported as null.
TRAFFIC = {
    "recall_decode": {"sources": ("recall_decode.hip", "recall.hpp", "stream.hpp", "common.hpp", "launch.hpp"),
                      "sha256": "ff5964b03e987cd2c290cbe854c0cb60f4f4132e8d48595fb6e60067d30df1c4",
                      "fetch_kib": 47205.0, "write_kib": 1274.4},
    "sparse_decode": {"sources": ("decode.hip", "stream.hpp", "common.hpp", "launch.hpp"),
                      "sha256": "8feced37d9113643b6d125b3ef6798e13c146b997b2591ef2bb70ee7f5084a6a",
                      "fetch_kib": 34286.7, "write_kib": 762.0},
}


def kernel_source_hash(sources) -> str:
    import hashlib

    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "semantic_cluster_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    t = TRAFFIC[kernel]
    if t["sha256"] is None or t["sha256"] != kernel_source_hash(t["sources"]):
        return None
    return t["fetch_kib"] * 1024 * 2.0 + t["write_kib"] * 1024 * 1.0


def copy_bandwidth(dev) -> float:
    """Measured device-to-device copy rate of 1 GiB (bytes read + written per second, GB/s):
    the practical HBM rate a streaming kernel can reach, reported beside the 8 TB/s peak."""
    import torch

    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 3 * 2 * src.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"[bench] device copy of 1 GiB: {gbs:.0f} GB/s (read + write)")
    return gbs


def run_cpu_baseline(cfg, steps: int, seconds: float = 20.0) -> dict:
    """The oracle, untuned, on the host cores: on every unit of the workload when
    it has at most 8 (timed in full), else on a bounded sample extrapolated to
    the workload's units."""
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
    units_total = cfg.layers * cfg.units
    full = units_total <= 8
    deadline = time.perf_counter() + (float("inf") if full else seconds)
    u = 0
    while time.perf_counter() < deadline and u < min(64, units_total):
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
    step_s = t_dec / n_unit_steps * units_total
    sample = (f"every unit ({n_units}) of the workload, {steps} decode steps each (select + decode, float64 "
              f"NumPy), and its whole prefill: timed in full" if full else
              f"{n_units} units x {steps} decode steps (select + decode, float64 NumPy) of the same "
              f"workload, extrapolated to {units_total} units per step; prefill of the same "
              f"{n_units} units timed for K-means keys/s")
    return {
        "value": cfg.batch / step_s,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": sample,
        "kmeans_keys_per_s": n_units * cfg.m / t_pre,
        "seconds": t_pre + t_dec,
    }


def incremental_bytes(units: int, K: int, m_old: int, m_new: int) -> int:
    """Algorithmic HBM bytes of one ckv_cluster_incremental call.

    Per unit: the new keys read twice (assignment, norms: 2 x 256 B each) and
    their labels written; every clustered token's label read twice (histogram,
    scatter) and its index written (4 + 4 + 4 B); every clustered token's K and
    V rows gathered and written in cluster order (4 x 256 B); per cluster the
    bf16 direction read and written, both f64 sums read and written, the f32
    mean written, the size read and written and the offset written.
    """
    d = 128
    m = m_old + m_new
    per_cluster = 2 * 2 * d + 2 * 2 * 8 * d + 4 * d + 4 * 2 + 4
    return units * (m_new * (2 * 2 * d + 4) + m * (4 + 4 + 4 + 4 * 2 * d) + K * per_cluster)


def split_bytes(units: int, K: int, m: int, split_rows: int) -> int:
    """Algorithmic HBM bytes of one ckv_cluster_split call.

    The split itself reads every cluster's f64 sum and size and, for each split
    cluster, its members' keys once (256 B per row; the seed search and the
    move both need them, but one read suffices) and their token ids, and
    writes their labels (4 + 4 B per row).  The rebuild that
    follows: labels read twice and the index written, K and V rows gathered
    and written in cluster order (each key's norm is taken from the row as it
    passes), and the per-cluster state rewritten.
    """
    d = 128
    per_cluster = 8 * d + 4 + 2 * 2 * d + 8 * d * 2 + 4 * d + 4 * 2 + 4
    split = split_rows * (2 * d + 4 + 4)
    rebuild = m * (4 + 4 + 4 + 4 * 2 * d)
    return units * (K * per_cluster + rebuild) + split


def split_plan(L, reserve: int):
    """Threshold for the split measurement (the median drift 1 - |S|/n over the
    clusters with at least two members) and the number of rows in the clusters
    it will split: per unit the min(reserve + already-empty slots, candidates)
    most drifted candidates.  Device tensors, outside the timed region."""
    import torch

    n = L.csize.to(torch.float64)
    drift = 1.0 - torch.linalg.vector_norm(L.csum, dim=-1) / n.clamp(min=1.0)
    ok = L.csize >= 2
    tau = float(drift[ok].median())
    cand = torch.where(ok & (drift > tau), drift, torch.full_like(drift, -1.0))
    free = (L.csize == 0).sum(dim=1)
    order = torch.argsort(cand, dim=1, descending=True)
    rank = torch.empty_like(order)
    rank.scatter_(1, order, torch.arange(order.shape[1], device=order.device).expand_as(order))
    take = (cand > tau) & (rank < free[:, None])
    rows = int((L.csize * take).sum())
    return tau, rows


def setup(args):
    import torch

    from semantic_cluster_sparse_amd import ckv

    ckv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return dev


def full_attention_baseline(layers, qs, qlast, outs, units, G, r_now, dec_ms, cs, stream, dev) -> dict:
    """Dense decode on the same harness: with budget >= m, ckv_select takes every
    cluster whole, so ckv_sparse_decode attends to every cached token.  Timed like
    the sparse decode (one graph over all layers, events around its replays)."""
    import torch

    n_layers = len(layers)
    m_now = layers[0].n_clustered - 16
    sp_full = [torch.empty((units, m_now), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    cnt_full = [torch.empty((units,), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    for li, L in enumerate(layers):
        L.select(qs[li][qlast], m_now, sp_full[li], cnt_full[li])

    def decode_full() -> None:
        for li, L in enumerate(layers):
            L.sparse_decode(qs[li][qlast], sp_full[li], cnt_full[li], m_now, outs[li])

    if cs is not None:
        fg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fg, stream=cs):
            decode_full()
        launch_full = fg.replay
    else:
        launch_full = decode_full
    launch_full()
    torch.cuda.synchronize()
    reps = 3
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        launch_full()
    b.record(stream)
    torch.cuda.synchronize()
    full_ms = a.elapsed_time(b) / (reps * n_layers)
    fbytes = decode_bytes(units, 16, m_now, r_now, G)
    gbs = fbytes / (full_ms * 1e-3) / 1e9
    log(f"[bench] full-attention decode {full_ms * 1e3:.1f} us/launch ({gbs:.0f} GB/s); "
        f"the sparse launch is {full_ms / dec_ms:.1f}x faster")
    return {"decode_us": full_ms * 1e3, "bytes_per_launch": fbytes, "achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
            "decode_speedup": full_ms / dec_ms}


def assign_flops(units: int, m: int, K: int) -> int:
    """Algorithmic flops of one assignment pass: 2 m K d per unit (the distance
    matmul; the argmax and padded directions are not counted)."""
    return 2 * units * m * K * 128


def time_assign(layers, cfg, units: int, stream) -> dict:
    """The assignment step alone (ckv_assign) on every layer after the prefill,
    between HIP events on the stream it runs on: one untimed pass over the
    layers, then one timed pass.  The labels are saved before and put back
    after, so the layers' state is the prefill's."""
    import torch

    saved = [L.assign.clone() for L in layers]
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for L in layers:
        L.assign_only(cfg.n_tokens)
    ea.record(stream)
    for L in layers:
        L.assign_only(cfg.n_tokens)
    eb.record(stream)
    torch.cuda.synchronize()
    for L, a in zip(layers, saved):
        L.assign.copy_(a)
    torch.cuda.synchronize()
    us = ea.elapsed_time(eb) * 1e3 / len(layers)
    flops = assign_flops(units, cfg.m, cfg.n_clusters)
    tf = flops / (us * 1e-6) / 1e12
    log(f"[bench] ckv_assign {us:.1f} us per layer ({flops / 1e9:.1f} GFLOP): {tf:.0f} TFLOP/s, "
        f"{tf / MFMA_BF16_PEAK_TFS:.3f} of the bf16 MFMA peak")
    kernel = "ckv::assign_resident_kernel" if cfg.n_clusters <= 512 else "ckv::assign_kernel"
    # keys through the assignment step per second (one pass per Lloyd round)
    keys_per_s = units * cfg.m / (us * 1e-6)
    return {"bound": "mfma", "kernel": kernel, "achieved": tf, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": tf / MFMA_BF16_PEAK_TFS, "launch_us": us, "flops_per_launch": flops,
            "keys_per_s": keys_per_s}


def run_stack(cfg, args) -> dict:
    """Decode steps through a layer stack (append_select + sparse_decode per layer),
    with ckv_cluster_incremental on every layer whenever 320 recent tokens have built up."""
    import torch

    from synth import device as dgen
    from semantic_cluster_sparse_amd.layer import Layer

    dev = setup(args)
    n_layers = args.layers or cfg.layers
    W = args.warmup
    K = args.steps if args.steps is not None else cfg.steps
    n_fill = cfg.n_tokens + cfg.n_recent
    cap = n_fill + W + K + 1
    units, G, budget = cfg.units, cfg.group, cfg.budget
    recluster = cfg.new_tokens if cfg.new_tokens > 0 else 0
    so = seed_offset(cfg)
    ph = bool(args.per_head_recall)
    fused = not args.separate
    stream = torch.cuda.current_stream()

    log(f"[bench] {cfg.name}: allocating {n_layers} layers of {units} units, capacity {cap}")
    layers = []
    qs = []
    for li in range(n_layers):
        L = Layer(batch=cfg.batch, n_kv_heads=cfg.n_kv_heads, group=G, n_clusters=cfg.n_clusters,
                  capacity=cap, max_budget=budget, incremental=recluster > 0, per_head=ph, device=dev)
        cen = dgen.fill_mixture(L.k_tok, L.v_tok, n_fill, cfg.components, seed=10_000 + so + li)
        qs.append([dgen.queries(cen, G, seed=20_000 + so + 100 * li + s) for s in range(W + K)])
        del cen
        layers.append(L)
    torch.cuda.synchronize()
    log(f"[bench] generated inputs; {torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    # ---------------------------------------------------------------- prefill (timed separately)
    # seeded prefill: the library draws each unit's initial indices (seed + unit); layers get disjoint seeds
    seeds = [30_000 + so + li * units for li in range(n_layers)]
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for li, L in enumerate(layers):
        L.prefill(cfg.n_tokens, cfg.iters, seeds[li])
    ev1.record(stream)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    prefill_ev_s = ev0.elapsed_time(ev1) / 1e3
    keys = n_layers * units * cfg.m
    log(f"[bench] prefill {prefill_s * 1e3:.1f} ms wall, {prefill_ev_s * 1e3:.1f} ms events; "
        f"{keys / prefill_ev_s / 1e6:.1f} M keys/s")
    assign = time_assign(layers, cfg, units, stream)
    # the recent tokens past the clustered prefix are already in the token-order rows
    for L in layers:
        L.set_counters(n_fill, cfg.n_tokens)

    # ---------------------------------------------------------------- decode step buffers
    sets = units * G if ph else units     # recalled sets per layer
    sel_pos = [torch.zeros((sets, budget), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    cnt = [torch.zeros((sets,), dtype=torch.int32, device=dev) for _ in range(n_layers)]
    outs = [torch.zeros((units, G, 128), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    k_new = [dgen.rows(units, 128, 40_000 + s, dev) for s in range(W + K)]
    v_new = [dgen.rows(units, 128, 50_000 + s, dev) for s in range(W + K)]
    incr_steps = []      # steps that start a re-clustering
    commit_steps = []    # asynchronous mode: steps before which the last layers are committed
    lag = args.async_lag if (recluster and args.async_recluster) else 0
    main = torch.cuda.current_stream()
    bs = torch.cuda.Stream() if lag else None          # background clustering stream
    starts = {}          # step -> layers whose clustering starts before it
    commits = {}         # step -> (layer, start step) committed before it
    bg_work = {}         # step -> graph of that step's background clustering
    bg_done = {}         # start step -> event on the background stream
    busy = [False]

    def nxt(li: int):
        """The layer whose call follows layer li's on the stream (the prefetch hint)."""
        return None if args.no_prefetch else layers[(li + 1) % n_layers]

    def recluster_due() -> bool:
        return bool(recluster) and layers[0].n_total - layers[0].n_clustered >= recluster

    def host_schedule(s: int) -> None:
        """Asynchronous mode.  When 320 recent tokens have built up, the layers'
        clusterings start spread over the first half of the next `lag` steps, and
        each is committed half a window after its start, so the background work
        is shared out over the steps instead of landing on one."""
        for li, _ in commits.get(s, []):
            layers[li].commit()
        if commits.get(s) and not any(t > s for t in commits):
            commit_steps.append(s)
            busy[0] = False
        if not busy[0] and recluster_due():
            busy[0] = True
            incr_steps.append(s)
            spread = max(1, lag // 2)
            for li in range(n_layers):
                st = s + (li * spread) // n_layers
                starts.setdefault(st, []).append(li)
                commits.setdefault(st + lag - spread, []).append((li, st))

    def background(s: int) -> None:
        for li in starts.get(s, []):
            layers[li].incremental_async()

    def step(s: int) -> None:
        if not lag and recluster_due():
            incr_steps.append(s)
            for L in layers:
                L.incremental()
        for li, L in enumerate(layers):
            if ph and fused:
                L.append(k_new[s], v_new[s])
                L.select_decode_per_head(qs[li][s], budget, sel_pos[li], cnt[li], outs[li], next_layer=nxt(li))
            elif ph:
                L.append(k_new[s], v_new[s])
                L.select_per_head(qs[li][s], budget, sel_pos[li], cnt[li])
                L.sparse_decode_per_head(qs[li][s], sel_pos[li], cnt[li], budget, outs[li])
            elif fused:
                L.append_select_decode(k_new[s], v_new[s], qs[li][s], budget, sel_pos[li], cnt[li], outs[li],
                                       next_layer=nxt(li))
            else:
                L.append_select(k_new[s], v_new[s], qs[li][s], budget, sel_pos[li], cnt[li])
                L.sparse_decode(qs[li][s], sel_pos[li], cnt[li], budget, outs[li])

    graphs = []
    cs = None
    if not args.no_graph:
        log("[bench] capturing one HIP graph per step")
        cs = torch.cuda.Stream()
        bcs = torch.cuda.Stream() if lag else None
        for s in range(W + K):
            if lag:
                host_schedule(s)
                if starts.get(s):
                    bg = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(bg, stream=bcs):
                        background(s)
                    bg_work[s] = bg
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                step(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(s: int) -> None:
        if lag:
            if not graphs:
                host_schedule(s)
            for st in sorted({st for _, st in commits.get(s, [])}):
                main.wait_event(bg_done[st])
            if starts.get(s):
                # the clustering reads the rows appended so far: start after the main stream's work
                ready = torch.cuda.Event()
                ready.record(main)
                bs.wait_event(ready)
                with torch.cuda.stream(bs):
                    if graphs:
                        bg_work[s].replay()
                    else:
                        background(s)
                    bg_done[s] = torch.cuda.Event()
                    bg_done[s].record(bs)
        if graphs:
            graphs[s].replay()
        else:
            step(s)

    for s in range(W):
        run(s)
    torch.cuda.synchronize()
    log("[bench] warmup done; timing")
    per_step = bool(recluster)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)] if per_step else []
    t0 = time.perf_counter()
    if per_step:
        evs[0].record(stream)
    for i, s in enumerate(range(W, W + K)):
        run(s)
        if per_step:
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / K * 1e3
    tokens_per_s = cfg.batch * K / dt
    log(f"[bench] {ms_per_step:.3f} ms/step, {tokens_per_s:.1f} tokens/s")

    # ---------------------------------------------------------------- kernel timing for the roofline
    # The priced kernel (the fused recall + decode, or ckv_sparse_decode in the
    # separate form) is one kernel per call.  The calls of all layers are
    # captured once more as a graph and replayed back to back between two
    # events on the stream they run on; the average is per launch.
    qlast = W + K - 1

    def decode_all() -> None:
        for li, L in enumerate(layers):
            if fused:
                (L.select_decode_per_head if ph else L.select_decode)(qs[li][qlast], budget, sel_pos[li], cnt[li],
                                                                      outs[li], next_layer=nxt(li))
            else:
                (L.sparse_decode_per_head if ph else L.sparse_decode)(qs[li][qlast], sel_pos[li], cnt[li], budget,
                                                                      outs[li])

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
    if ph:
        # The heads of one KV head recall overlapping sets, and their shared rows
        # are fetched from HBM once (the rest hit the caches), so the bytes that
        # must move are those of each unit's union of recalled rows, plus every
        # set's indices and every head's query and output.
        srt = sel_pos[n_layers - 1].view(units, G * budget).sort(dim=1).values
        distinct = int((1 + (srt[:, 1:] != srt[:, :-1]).sum(dim=1)).sum())
        dbytes = (units * (16 + r_now) + distinct) * 2 * 128 * 2 + sets * (4 * budget + 2 * 128 + 4 * 128)
        if fused:
            # every set's recall reads its unit's centroids and offsets (once per unit
            # from HBM: the sets of a unit share them through the caches), writes its
            # count and scores its cut cluster's unkept tokens
            dbytes += units * (4 * cfg.n_clusters * 128 + 4 * (cfg.n_clusters + 1)) + sets * (
                4 + CUT_UNKEPT_ROWS * 2 * 128)
        log(f"[bench] per-head recall: {distinct / units:.0f} distinct recalled rows per unit "
            f"(of {G * budget} recalled)")
    elif fused:
        dbytes = fused_bytes(units, 16, budget, r_now, G, cfg.n_clusters)
    else:
        dbytes = decode_bytes(units, 16, budget, r_now, G)
    achieved = dbytes / (dec_ms * 1e-3) / 1e9
    r_mean = cfg.n_recent + (W + K) // 2
    if recluster:
        r_mean = recluster // 2
    if ph:
        step_bytes = n_layers * (decode_bytes(sets, 16, budget, r_mean, 1)
                                 + select_bytes(sets, cfg.n_clusters, budget, 1, 82) + units * 2 * 256)
    elif fused:
        step_bytes = n_layers * (fused_bytes(units, 16, budget, r_mean, G, cfg.n_clusters) + units * 2 * 256)
    else:
        step_bytes = n_layers * (decode_bytes(units, 16, budget, r_mean, G)
                                 + select_bytes(units, cfg.n_clusters, budget, G, 82) + units * 2 * 256)
    priced = "ckv_select_decode" if fused else "ckv_sparse_decode"
    log(f"[bench] {priced}{'_per_head' if ph else ''} {dec_ms * 1e3:.1f} us/launch, {achieved:.0f} GB/s algorithmic")

    # ---------------------------------------------------------------- full-attention baseline
    full = None
    if not args.no_full_attention:
        full = full_attention_baseline(layers, qs, qlast, outs, units, G, r_now, dec_ms, cs if graphs else None,
                                       stream, dev)
        full["step_speedup"] = n_layers * full["decode_us"] * 1e-3 / ms_per_step
    # counters taken on the default workload (the fused form with the next layer's
    # centroids read at the end of each launch, which they include)
    traffic = (measured_traffic("recall_decode" if fused else "sparse_decode")
               if cfg.name == DEFAULT_WORKLOAD and n_layers == cfg.layers and not ph
               and not (fused and args.no_prefetch) else None)
    copy_gbs = copy_bandwidth(dev)

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
                   "group": G, "context": n_fill, "clusters": cfg.n_clusters, "budget": budget,
                   "graphs": not args.no_graph, "recall": "per query head" if ph else "per KV head (summed query)",
                   "launches_per_layer": ("2 (ckv_append + ckv_select_decode_per_head)" if ph else "1") if fused
                   else ("3" if ph else "2 (ckv_append_select + ckv_sparse_decode)"),
                   "prefetch_next_layer": fused and not args.no_prefetch},
        "roofline": {"bound": "hbm",
                     "kernel": f"ckv::{'recall_decode_kernel' if fused else 'sparse_decode_kernel'}"
                               f"<{1 if ph else _group_tier(G)}>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "launch_us": dec_ms * 1e3, "bytes_per_launch": dbytes,
                     "copy_gbs": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        "step_hbm_frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kmeans_keys_per_s": keys / prefill_ev_s,
        "prefill_ms": prefill_ev_s * 1e3,
        "assign_roofline": assign,
        "full_attention": full,
    }
    if per_step:
        times = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
        timed_incr = [s - W for s in incr_steps if W <= s < W + K]
        timed_commit = [s - W for s in commit_steps if W <= s < W + K]
        # steps that carry re-clustering work: the step itself (synchronous), or every
        # step from the start to the commit (asynchronous, the work overlaps them)
        carry = set(timed_incr)
        for a0 in timed_incr:
            ends = [c for c in timed_commit if c > a0]
            if lag and ends:
                carry.update(range(a0, ends[0] + 1))
        window = sorted(carry)
        plain = sorted(t for i, t in enumerate(times) if i not in carry)
        t_plain = plain[len(plain) // 2] if plain else float("nan")
        extra = sum(times[i] - t_plain for i in carry)
        n_done = len(timed_commit) if lag else len(timed_incr)
        result["recluster"] = {
            "every_tokens": recluster,
            "mode": (f"async: layers start over {max(1, lag // 2)} steps, each committed "
                     f"{lag - max(1, lag // 2)} steps after its start") if lag else "sync",
            "steps_with_recluster": timed_incr,
            "commit_steps": timed_commit,
            "step_ms_median": t_plain,
            "step_ms_max": max(times),
            "window_step_ms": [round(times[i], 3) for i in window],
            "recluster_ms": extra,
            "steady_tokens_per_s": (cfg.batch / ((t_plain + extra / n_done / recluster) * 1e-3)
                                    if n_done else None),
        }
        log(f"[bench] median step {t_plain:.3f} ms, slowest {max(times):.3f} ms; re-clustering started at "
            f"{timed_incr}, committed at {timed_commit}: {extra:.3f} ms extra over those steps")
    return result


def run_incremental(cfg, args) -> dict:
    """One layer: prefill, append cfg.new_tokens keys per unit, then time
    ckv_cluster_incremental, ckv_select and ckv_sparse_decode, and the fused
    ckv_select_decode (median over repetitions)."""
    import torch

    from synth import device as dgen
    from semantic_cluster_sparse_amd.layer import Layer

    dev = setup(args)
    W = args.warmup
    reps = args.steps if args.steps is not None else 10
    n0, n_new = cfg.n_tokens, cfg.new_tokens
    units, G, budget = cfg.units, cfg.group, cfg.budget
    cap = n0 + n_new
    so = seed_offset(cfg)
    stream = torch.cuda.current_stream()
    R = args.split_reserve
    L = Layer(batch=cfg.batch, n_kv_heads=cfg.n_kv_heads, group=G, n_clusters=cfg.n_clusters + R,
              capacity=cap, max_budget=budget, incremental=True, device=dev)
    cen = dgen.fill_mixture(L.k_tok, L.v_tok, n0, cfg.components, seed=10_000 + so)
    k_add, v_add = dgen.new_rows(cen, n_new, cfg.new_components, cfg.new_fraction,
                                 seed=60_000 + so)
    q = dgen.queries(cen, G, seed=20_000 + so)
    init = dgen.init_indices(units, cfg.m, cfg.n_clusters, seed=30_000 + so, device=dev)
    if R:
        # slots held empty at prefill (init index -1) for the drift split to fill
        init = torch.cat([init, torch.full((units, R), -1, dtype=torch.int32, device=dev)], 1).contiguous()
    del cen
    sel_pos = torch.zeros((units, budget), dtype=torch.int32, device=dev)
    cnt = torch.zeros((units,), dtype=torch.int32, device=dev)
    out = torch.zeros((units, G, 128), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: {units} units, {n0} clustered + {n_new} new tokens; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    t_inc, t_sel, t_dec, t_sel0, t_split, split_rows, t_fused = [], [], [], [], [], [], []
    for r in range(W + reps):
        L.prefill(n0, cfg.iters, init)
        L.k_tok[:, n0:cap].copy_(k_add)
        L.v_tok[:, n0:cap].copy_(v_add)
        L.set_counters(cap, n0)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        torch.cuda.synchronize()
        e[0].record(stream)
        L.select(q, budget, sel_pos, cnt)        # recall with the 320 tokens still recent
        e[1].record(stream)
        L.incremental()
        e[2].record(stream)
        L.select(q, budget, sel_pos, cnt)
        e[3].record(stream)
        L.sparse_decode(q, sel_pos, cnt, budget, out)
        e[4].record(stream)
        L.select_decode(q, budget, sel_pos, cnt, out)  # the same recall and attention in one launch
        e[5].record(stream)
        torch.cuda.synchronize()
        if R:
            tau, rows = split_plan(L, R)
            es = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            es[0].record(stream)
            L.split(tau)
            es[1].record(stream)
            torch.cuda.synchronize()
            if r >= W:
                t_split.append(es[0].elapsed_time(es[1]))
                split_rows.append(rows)
        if r >= W:
            t_sel0.append(e[0].elapsed_time(e[1]))
            t_inc.append(e[1].elapsed_time(e[2]))
            t_sel.append(e[2].elapsed_time(e[3]))
            t_dec.append(e[3].elapsed_time(e[4]))
            t_fused.append(e[4].elapsed_time(e[5]))

    def med(x):
        return sorted(x)[len(x) // 2]

    inc_ms = med(t_inc)
    copy_gbs = copy_bandwidth(dev)
    ibytes = incremental_bytes(units, cfg.n_clusters, cfg.m, n_new)
    achieved = ibytes / (inc_ms * 1e-3) / 1e9
    log(f"[bench] ckv_cluster_incremental {inc_ms * 1e3:.1f} us, {achieved:.0f} GB/s algorithmic; "
        f"select {med(t_sel) * 1e3:.1f} us; decode {med(t_dec) * 1e3:.1f} us; fused recall + decode "
        f"{med(t_fused) * 1e3:.1f} us")
    extra = {}
    if R:
        sp_ms = med(t_split)
        rows = split_rows[0]
        sbytes = split_bytes(units, L.n_clusters, cfg.m + n_new, rows)
        extra["split"] = {"reserved_slots": R, "threshold": "median drift of the clusters with >= 2 members",
                          "us": sp_ms * 1e3, "candidate_rows": rows, "bytes": sbytes,
                          "achieved_gbs": sbytes / (sp_ms * 1e-3) / 1e9,
                          "frac": sbytes / (sp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[bench] ckv_cluster_split {sp_ms * 1e3:.1f} us ({R} reserved slots per unit, "
            f"{rows} rows in split clusters), {extra['split']['achieved_gbs']:.0f} GB/s algorithmic")
    return {
        "metric": "incremental clustering latency (320 new keys per KV head), then budget-1024 recall",
        "value": inc_ms * 1e3,
        "unit": "us",
        "n_gpus": 1,
        "steps": reps,
        "warmup": W,
        "ms_per_step": inc_ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": 1, "batch": cfg.batch, "kv_heads": cfg.n_kv_heads,
                   "group": G, "context": n0, "new_tokens": n_new, "new_components": cfg.new_components,
                   "new_fraction": cfg.new_fraction, "clusters": cfg.n_clusters, "budget": budget},
        "roofline": {"bound": "hbm", "kernel": "ckv_cluster_incremental (whole call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "launch_us": inc_ms * 1e3, "bytes_per_launch": ibytes,
                     "copy_gbs": copy_gbs, "frac_of_copy": achieved / copy_gbs},
        "select_us": med(t_sel) * 1e3,
        "select_before_incremental_us": med(t_sel0) * 1e3,
        "sparse_decode_us": med(t_dec) * 1e3,
        "select_decode_us": med(t_fused) * 1e3,
        **extra,
    }


def run_cpu_baseline_incremental(cfg, seconds: float = None) -> dict:
    """The oracle's incremental pass (the same 320 new keys per unit, 10% from 8
    new components) on every unit of the workload (seconds=None), each after its
    own oracle prefill (untimed; about 2 s per unit), or on the units that fit in
    `seconds`, extrapolated to the workload's units."""
    import numpy as np

    import synth
    from oracle import pipeline

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    t_inc = 0.0
    n_units = 0
    deadline = time.perf_counter() + seconds if seconds is not None else float("inf")
    n_new = cfg.n_tokens + cfg.new_tokens
    while time.perf_counter() < deadline and n_units < cfg.units:
        u = n_units
        k, v, cen = synth.make_layer_inputs(cfg, units=[u], capacity=n_new)
        kn, vn, _ = synth.make_new_tokens(cfg.data_seed, cen, cfg.new_tokens, cfg.new_components, cfg.new_fraction,
                                          unit_ids=[u])
        k[:, cfg.n_tokens:n_new] = kn
        v[:, cfg.n_tokens:n_new] = vn
        init = synth.make_init_indices(cfg.init_seed, 1, cfg.m, cfg.n_clusters, unit_ids=[u])[0]
        st = pipeline.prefill_unit(k[0], cfg.n_tokens, init, cfg.n_clusters, cfg.iters, v_bits=v[0])
        t0 = time.perf_counter()
        pipeline.incremental_unit(st, k[0], n_new, v_bits=v[0])
        t_inc += time.perf_counter() - t0
        n_units += 1
    us = t_inc / n_units * cfg.units * 1e6
    return {"value": us, "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": (f"the incremental pass of every unit ({n_units}), each after its own untimed oracle prefill, "
                       f"float64 NumPy: timed in full" if n_units == cfg.units else
                       f"the incremental pass of {n_units} units (each after its own untimed oracle prefill), "
                       f"float64 NumPy, extrapolated to {cfg.units} units"),
            "seconds": t_inc}


def seed_offset(cfg) -> int:
    """Generator seeds of a workload: the default one keeps offset 0, the others get their own range."""
    return 0 if cfg.name == DEFAULT_WORKLOAD else 100_000 * cfg.seed_base


def _group_tier(G: int) -> int:
    t = 1
    while t < G:
        t <<= 1
    return t


DEFAULT_WORKLOAD = "llama8b-stack-32k-b8"
WORKLOADS = (DEFAULT_WORKLOAD, "glm4-stack-32k-b16", "llama8b-incremental-b16", "single-head-2k",
             "llama8b-layer-32k")
# decode steps timed on the single-layer workloads when --steps is not given
SINGLE_LAYER_STEPS = 200


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 for the default workload, the workload's own count otherwise)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", choices=WORKLOADS, default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (debug only)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-attention", action="store_true", help="skip the dense-decode baseline")
    ap.add_argument("--async-recluster", action="store_true",
                    help="re-cluster on a second stream beside the decode steps and commit later")
    ap.add_argument("--async-lag", type=int, default=16, help="steps between starting and committing")
    ap.add_argument("--per-head-recall", action="store_true",
                    help="one recall and attention set per query head instead of per KV head")
    ap.add_argument("--no-prefetch", action="store_true",
                    help="fused form: do not pass the next layer as the centroid prefetch hint")
    ap.add_argument("--separate", action="store_true",
                    help="recall and decode as two launches per layer (ckv_append_select + ckv_sparse_decode) "
                         "instead of the fused ckv_append_select_decode")
    ap.add_argument("--split-reserve", type=int, default=0,
                    help="llama8b-incremental-b16 only: hold this many cluster slots empty at prefill and "
                         "time ckv_cluster_split after the incremental call")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="bound on the oracle's timed work (default: 20 s on the stacks; every unit of the "
                         "one-layer and incremental workloads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 1 GiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by unit with no exchange between GPUs)", file=sys.stderr)
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

    cfg = synth.CONFIGS[args.workload]
    if args.workload == DEFAULT_WORKLOAD and args.steps is None:
        args.steps = 20
    if cfg.layers == 1 and not cfg.new_tokens and args.steps is None:
        args.steps = SINGLE_LAYER_STEPS
    if cfg.new_tokens and cfg.layers == 1:
        result = run_incremental(cfg, args)
    else:
        result = run_stack(cfg, args)
    if not args.no_cpu_baseline and not args.per_head_recall and args.workload != "glm4-stack-32k-b16":
        log("[bench] timing the oracle on the host")
        if cfg.new_tokens and cfg.layers == 1:
            result["cpu_baseline"] = run_cpu_baseline_incremental(cfg, seconds=args.cpu_seconds)
        else:
            result["cpu_baseline"] = run_cpu_baseline(cfg, steps=3, seconds=args.cpu_seconds or 20.0)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
