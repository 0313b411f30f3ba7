"""GPU parity: libckv.so against the float64 oracle on identical bf16 inputs.

Bars (from the method's precision contract):
* assignments: bit-exact wherever the oracle's top-2 margin exceeds 1e-4 of
  |x| (teacher-forced: zero unexcused mismatches; end-to-end: at most 0.1%
  differing labels);
* centroid directions: bitwise equal to the oracle's bf16 values whenever
  the labels that produced them are equal;
* recall: the same token set wherever the oracle's boundary scores are more
  than 1e-4 (relative) apart; at most 0.1% of recalled tokens differ;
* decode: max |GPU - oracle| <= 2e-3 per output element.
Teacher-forced cases load the oracle's state into the GPU buffers; GPU
results are never fed back to the oracle.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import (DECODE_ATOL, MISMATCH_FRACTION, check_decode, check_state, compare_assign,
                      compare_selection, dev_bf16, gpu_layer, host_bits, load_state, say, to_dev)
from oracle import bf16, pipeline

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

from semantic_cluster_sparse_amd.layer import Layer  # noqa: E402

D = 128

# ------------------------------------------------------------------ prefill


def test_prefill_single_head_rounds():
    cfg = synth.CONFIGS["single-head-2k"]
    say(f"case: prefill {cfg.name}")
    k, v, _ = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, 1, cfg.m, cfg.n_clusters)
    ora = pipeline.prefill_unit(k[0], cfg.n_tokens, init[0], cfg.n_clusters, cfg.iters,
                                v_bits=v[0], history=True)
    x = bf16.widen(k[0][16:cfg.n_tokens])
    for T in (1, 2, 3, 5, 10):
        L = gpu_layer(k, v, 1, cfg.n_clusters)
        L.prefill(cfg.n_tokens, T, to_dev(init, torch.int32))
        torch.cuda.synchronize()
        a_o, c_o = ora["history"][T]
        st = dict(assign=a_o, cdir_bits=bf16.round_rne(c_o))
        if T == cfg.iters:
            st = ora
        else:
            from oracle import kmeans
            S, M, n = kmeans.unit_sums(x, a_o, cfg.n_clusters)
            perm, off = kmeans.build_index(a_o, cfg.n_clusters)
            st.update(csum=S, msum=M, csize=n, offsets=off, perm=perm,
                      cmean=kmeans.scoring_centroids(M, n), k_clu_bits=k[0][perm], v_clu_bits=v[0][perm])
        assert check_state(L, 0, st, x, ora["history"][T - 1][1], tag=f"T={T}") == 0
        assert L.n_total == cfg.n_tokens and L.n_clustered == cfg.n_tokens


def test_teacher_forced_lloyd_rounds():
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    say("case: teacher-forced Lloyd rounds, Llama layer shape, units 0-1")
    k, v, _ = synth.make_layer_inputs(cfg, units=[0, 1])
    init = synth.make_init_indices(cfg.init_seed, 2, cfg.m, cfg.n_clusters)
    oras = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, 4, v_bits=v[u],
                                  history=True) for u in range(2)]
    xs = [bf16.widen(k[u][16:cfg.n_tokens]) for u in range(2)]
    from oracle import kmeans
    for t in (1, 2, 4):
        L = gpu_layer(k, v, cfg.group, cfg.n_clusters)
        for u in range(2):
            L.cdir[u].copy_(dev_bf16(bf16.round_rne(oras[u]["history"][t - 1][1])))
        L.set_counters(cfg.n_tokens, 16)          # nothing clustered yet: one incremental = one round
        L.incremental()
        torch.cuda.synchronize()
        for u in range(2):
            a_o, c_o = oras[u]["history"][t]
            S, M, n = kmeans.unit_sums(xs[u], a_o, cfg.n_clusters)
            perm, off = kmeans.build_index(a_o, cfg.n_clusters)
            st = dict(assign=a_o, cdir_bits=bf16.round_rne(c_o), csum=S, msum=M, csize=n,
                      offsets=off, perm=perm, cmean=kmeans.scoring_centroids(M, n),
                      k_clu_bits=k[u][perm], v_clu_bits=v[u][perm])
            assert check_state(L, u, st, xs[u], oras[u]["history"][t - 1][1], tag=f"t={t}") == 0


@pytest.mark.parametrize("K", [400, 23, 700])
def test_assign_entry_teacher_forced(K):
    """ckv_assign alone: labels of every clustered key against oracle directions
    (a ragged last direction block at K = 23; the LDS-chunked kernel at K = 700),
    to the assignment bar."""
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    say(f"case: ckv_assign teacher-forced, Llama layer shape, K = {K}, units 0-1")
    k, v, _ = synth.make_layer_inputs(cfg, units=[0, 1])
    init = synth.make_init_indices(cfg.init_seed, 2, cfg.m, K)
    from oracle import kmeans
    L = gpu_layer(k, v, cfg.group, K)
    dirs = []
    for u in range(2):
        xs = bf16.widen(k[u][16:cfg.n_tokens])
        c = kmeans.init_directions(xs, init[u], K)
        dirs.append((xs, c))
        L.cdir[u].copy_(dev_bf16(bf16.round_rne(c)))
    L.assign.fill_(-7)
    L.assign_only(cfg.n_tokens)
    torch.cuda.synchronize()
    for u, (xs, c) in enumerate(dirs):
        a_o = kmeans.assign(xs, c)
        a_g = L.assign[u, :cfg.m].cpu().numpy()
        mism, unexc = compare_assign(a_g, a_o, xs, c)
        say(f"  unit {u}: label mismatches {mism} (unexcused {unexc}) of {cfg.m}")
        assert unexc == 0 and mism <= MISMATCH_FRACTION * cfg.m
    assert int((L.assign[:, cfg.m:] != -7).sum()) == 0, "ckv_assign wrote past the clustered tokens"


def test_llama_layer_end_to_end():
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    say(f"case: end-to-end {cfg.name}")
    k, v, cen = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    qd = dev_bf16(q)
    sel_pos = torch.zeros((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((cfg.units, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    total_mism = total_diff = compared = 0
    for u in (0, 3, 7):
        ora = pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=v[u],
                                    history=True)
        x = bf16.widen(k[u][16:cfg.n_tokens])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], tag="e2e")
        total_mism += mism
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, cfg.budget)
        total_diff += diff
        compared += check_decode(og[u], q[u], k[u], v[u], ora, sp[u], cn[u], sel, diff, 16, cfg.n_tokens,
                                 cfg.n_tokens, tag=f"unit {u}:")
    assert total_mism <= MISMATCH_FRACTION * 3 * cfg.m
    assert total_diff <= MISMATCH_FRACTION * 2 * 3 * cfg.budget
    assert compared >= 1, "no sampled unit's decode was compared"


def _random_case(rng):
    U = int(rng.integers(1, 4))
    n_sink = int(rng.choice([0, 5, 16]))
    K = int(rng.integers(1, 97))
    m = int(rng.integers(max(K, 40), 5001))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    T = int(rng.choice([1, 3]))
    u01 = rng.random()
    budget = 0 if u01 < 0.15 else (m + 7 if u01 > 0.85 else int(rng.integers(1, m + 1)))
    r = int(rng.integers(0, 41))
    C = int(rng.integers(4, 65))
    return U, n_sink, K, m, G, T, budget, r, C


@pytest.mark.parametrize("case", range(8))
def test_random_shapes_end_to_end(case):
    """Seeded random shapes (units, sinks, K, m, G, rounds, budget, recent rows,
    mixture size) through prefill, recall and decode, against the oracle; the
    last tile, direction block, chunk and position segment are ragged."""
    rng = np.random.default_rng(9000 + case)
    U, n_sink, K, m, G, T, budget, r, C = _random_case(rng)
    n = n_sink + m
    say(f"case {case}: units {U}, n_sink {n_sink}, K {K}, m {m}, G {G}, rounds {T}, budget {budget}, "
        f"recent {r}, components {C}")
    parts = [synth.make_unit_inputs(9100 + case, u, n + r, C) for u in range(U)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(9200 + case, U, m, K)
    q = synth.make_queries(9300 + case, cen, G)
    L = gpu_layer(k, v, G, K, n_sink=n_sink, max_budget=max(budget, 1))
    L.prefill(n, T, to_dev(init, torch.int32))
    L.set_counters(n + r, n)
    qd = dev_bf16(q)
    sel_pos = torch.zeros((U, max(budget, 1)), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((U,), dtype=torch.int32, device="cuda")
    out = torch.zeros((U, G, D), dtype=torch.float32, device="cuda")
    L.select(qd, budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, budget, out)
    torch.cuda.synchronize()
    sp = sel_pos.cpu().numpy()[:, :budget]
    cn, og = cnt.cpu().numpy(), out.cpu().numpy()
    total_mism = compared = 0
    for u in range(U):
        ora = pipeline.prefill_unit(k[u], n, init[u], K, T, n_sink=n_sink, v_bits=v[u], history=True)
        x = bf16.widen(k[u][n_sink:n])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], n_sink=n_sink, tag=f"case {case}")
        total_mism += mism
        if mism:
            continue
        assert int(cn[u]) == min(budget, m)
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, sp[u], cn[u], sel, diff, n_sink, n, n + r,
                                 tag=f"unit {u}:")
    assert total_mism <= max(1, MISMATCH_FRACTION * U * m)
    assert compared >= 1, "no unit's decode was compared"


@pytest.mark.parametrize("K", [700, 1024])
def test_large_k_end_to_end(K):
    # K > 512 takes the LDS-chunked assignment kernel; 1024 is the largest K the library accepts
    n, units, iters, budget, G = 16 + 24000, 2, 3, 2048, 4
    say(f"case: K={K} end to end, {units} units, n={n}, {iters} rounds, budget {budget}")
    ks, vs, cs = [], [], []
    for u in range(units):
        kb, vb, c = synth.make_unit_inputs(95, u, n, 1024)
        ks.append(kb), vs.append(vb), cs.append(c)
    k, v, cen = np.stack(ks), np.stack(vs), np.stack(cs)
    init = synth.make_init_indices(96, units, n - 16, K)
    q = synth.make_queries(97, cen, G)
    L = gpu_layer(k, v, G, K, max_budget=budget)
    L.prefill(n, iters, to_dev(init, torch.int32))
    sel_pos = torch.zeros((units, budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((units, G, D), dtype=torch.float32, device="cuda")
    qd = dev_bf16(q)
    L.select(qd, budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, budget, out)
    torch.cuda.synchronize()
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in range(units):
        ora = pipeline.prefill_unit(k[u], n, init[u], K, iters, v_bits=v[u], history=True)
        x = bf16.widen(k[u][16:n])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], tag=f"K={K}")
        assert mism <= MISMATCH_FRACTION * (n - 16)
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], budget)
        if compare_selection(L, u, sp, cn, ora, sel, budget) == 0:
            ref = pipeline.decode_unit(q[u], k[u], v[u], ora["k_clu_bits"], ora["v_clu_bits"], sel["positions"],
                                       16, n, n)
            err = np.abs(og[u] - ref).max()
            say(f"  unit {u}: decode max abs err {err:.3g}")
            assert err <= DECODE_ATOL
            compared += 1
    assert compared >= 1


# ------------------------------------------------------------------ select


def test_select_teacher_forced():
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    say("case: teacher-forced recall, Llama layer shape")
    units = [0, 1, 2, 3]
    k, v, cen = synth.make_layer_inputs(cfg, units=units)
    init = synth.make_init_indices(cfg.init_seed, len(units), cfg.m, cfg.n_clusters)
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, 2, v_bits=v[u])
              for u in range(len(units))]
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.m + 5)
    load_state(L, states)
    L.set_counters(cfg.n_tokens, cfg.n_tokens)
    qd = dev_bf16(q)
    for budget in (0, 1, 100, 1024, 4096, cfg.m, cfg.m + 5):
        sel_pos = torch.full((len(units), max(budget, 1)), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((len(units),), dtype=torch.int32, device="cuda")
        L.select(qd, budget, sel_pos, cnt)
        torch.cuda.synchronize()
        sp, cn = sel_pos.cpu().numpy(), cnt.cpu().numpy()
        for u in range(len(units)):
            st = states[u]
            mu32 = st["cmean"].astype(np.float32).astype(np.float64)
            sel = pipeline.select_unit(q[u], mu32, st["csize"], st["offsets"], st["k_clu_bits"], budget)
            c = min(budget, cfg.m)
            assert cn[u] == c
            pos_g = sp[u, :c]
            if not np.array_equal(pos_g, sel["positions"]):
                gap = selection_boundary_gap(sel, bf16.widen(st["k_clu_bits"]), st["offsets"])
                nd = len(set(pos_g.tolist()) ^ set(sel["positions"].tolist()))
                say(f"  budget {budget} unit {u}: {nd} positions differ, boundary gap {gap:.3g}")
                assert gap <= SELECT_GAP
        say(f"  budget {budget}: ok")


@pytest.mark.parametrize("U,iters", [(64, 2), (64, 7), (5, 4)])
def test_rounds_by_changes(U, iters):
    # The prefill's rounds between the first and the last move the cluster sums by the keys
    # that changed cluster.  64 units: one workgroup per (unit, 32-dim slice), a unit's
    # workgroups on one XCD; 5 units: ranges of clusters, no XCD mapping.  The oracle sums
    # every round from scratch, so the final state checks every round's update.
    K, n = 96, 16 + 6000
    say(f"case: rounds by changes, {U} units, K={K}, n={n}, {iters} rounds")
    ks, vs = [], []
    for u in range(U):
        kb, vb, _ = synth.make_unit_inputs(171, u, n, 128)
        ks.append(kb), vs.append(vb)
    k, v = np.stack(ks), np.stack(vs)
    init = synth.make_init_indices(172, U, n - 16, K)
    L = gpu_layer(k, v, 4, K, max_budget=256)
    L.prefill(n, iters, to_dev(init, torch.int32))
    torch.cuda.synchronize()
    moved = 0
    for u in sorted({0, U // 2, U - 1}):
        ora = pipeline.prefill_unit(k[u], n, init[u], K, iters, v_bits=v[u], history=True)
        hist = ora["history"]
        # keys that changed cluster in the rounds by changes (rounds 2 .. iters - 1)
        moved += sum(int((hist[t][0] != hist[t - 1][0]).sum()) for t in range(2, iters))
        x = bf16.widen(k[u][16:n])
        assert check_state(L, u, ora, x, hist[-2][1], tag=f"U={U} T={iters}") == 0
    if iters > 2:
        assert moved > 0, "no key changed cluster in the rounds by changes"


@pytest.mark.parametrize("shape", ["llama8b-layer-32k", "glm4-stack-32k-b16"])
def test_per_head_recall_and_decode(shape):
    """Per-query-head recall + decode, teacher-forced: the Llama layer (G = 4, units 0-3,
    budget 1024) and the GLM4-shaped layer (G = 16, 410 clusters, 300 recent rows, units
    0-1, budget 2048)."""
    cfg = synth.CONFIGS[shape]
    budget = 1024 if shape.startswith("llama") else cfg.budget
    units = [0, 1, 2, 3] if shape.startswith("llama") else [0, 1]
    n_all = cfg.n_tokens + cfg.n_recent
    say(f"case: per-query-head recall + decode, {shape}, units {units}, G={cfg.group}, budget {budget}, "
        f"{cfg.n_recent} recent rows")
    U = len(units)
    k, v, cen = synth.make_layer_inputs(cfg, units=units)
    init = synth.make_init_indices(cfg.init_seed, U, cfg.m, cfg.n_clusters)
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, 2, v_bits=v[u])
              for u in range(U)]
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    Lh = Layer(batch=U, n_kv_heads=1, group=cfg.group, n_clusters=cfg.n_clusters, capacity=k.shape[1],
               max_budget=budget, incremental=False, per_head=True)
    Lh.k_tok.copy_(dev_bf16(k))
    Lh.v_tok.copy_(dev_bf16(v))
    load_state(Lh, states)
    Lh.set_counters(n_all, cfg.n_tokens)
    qd = dev_bf16(q)
    S = U * cfg.group
    sel_pos = torch.full((S, budget), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((S,), dtype=torch.int32, device="cuda")
    out = torch.zeros((U, cfg.group, D), dtype=torch.float32, device="cuda")
    Lh.select_per_head(qd, budget, sel_pos, cnt)
    Lh.sparse_decode_per_head(qd, sel_pos, cnt, budget, out)
    torch.cuda.synchronize()
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    assert np.all(cn == budget)
    distinct = 0
    for u in range(U):
        st = states[u]
        mu32 = st["cmean"].astype(np.float32).astype(np.float64)
        sels = pipeline.select_per_head(q[u], mu32, st["csize"], st["offsets"], st["k_clu_bits"], budget)
        ok = True
        for g in range(cfg.group):
            pos_g = sp[u * cfg.group + g, :budget]
            assert np.all(np.diff(pos_g) > 0)
            if not np.array_equal(pos_g, sels[g]["positions"]):
                gap = selection_boundary_gap(sels[g], bf16.widen(st["k_clu_bits"]), st["offsets"])
                say(f"  unit {u} head {g}: recall differs, boundary gap {gap:.3g}")
                assert gap <= SELECT_GAP
                ok = False
        distinct += len({tuple(x["positions"].tolist()) for x in sels}) > 1
        if ok:
            ref = pipeline.decode_per_head(q[u], k[u], v[u], st["k_clu_bits"], st["v_clu_bits"],
                                           [x["positions"] for x in sels], 16, cfg.n_tokens, n_all)
            err = np.abs(og[u] - ref).max()
            say(f"  unit {u}: per-head decode max abs err {err:.3g}")
            assert err <= DECODE_ATOL
    assert distinct > 0, "the heads of every unit recalled the same set: the case does not exercise the mode"


def test_per_head_after_prefill_many_units():
    # 64 units x 4 heads: the per-head arrival counters reach past the per-KV-head ones, and the
    # prefill on the same workspace must not disturb them (every set must come back full)
    U, G, K, n, budget, iters = 64, 4, 40, 16 + 3000, 512, 2
    say(f"case: per-query-head recall after a prefill on the same workspace, {U} units x {G} heads")
    ks, vs, cs = [], [], []
    for u in range(U):
        kb, vb, c = synth.make_unit_inputs(131, u, n, 48)
        ks.append(kb), vs.append(vb), cs.append(c)
    k, v, cen = np.stack(ks), np.stack(vs), np.stack(cs)
    init = synth.make_init_indices(132, U, n - 16, K)
    q = synth.make_queries(133, cen, G)
    L = Layer(batch=U, n_kv_heads=1, group=G, n_clusters=K, capacity=n, max_budget=budget, incremental=False,
              per_head=True)
    L.k_tok.copy_(dev_bf16(k))
    L.v_tok.copy_(dev_bf16(v))
    L.prefill(n, iters, to_dev(init, torch.int32))
    sel_pos = torch.full((U * G, budget), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((U * G,), dtype=torch.int32, device="cuda")
    out = torch.zeros((U, G, D), dtype=torch.float32, device="cuda")
    qd = dev_bf16(q)
    for _ in range(2):              # twice: the counters must come back to zero
        L.select_per_head(qd, budget, sel_pos, cnt)
        L.sparse_decode_per_head(qd, sel_pos, cnt, budget, out)
    torch.cuda.synchronize()
    cn, sp, og = cnt.cpu().numpy(), sel_pos.cpu().numpy(), out.cpu().numpy()
    assert np.all(cn == budget), f"{int((cn != budget).sum())} sets came back short"
    assert np.all(np.diff(sp, axis=1) > 0)
    for u in (0, 37, 63):
        ora = pipeline.prefill_unit(k[u], n, init[u], K, iters, v_bits=v[u], history=True)
        x = bf16.widen(k[u][16:n])
        if check_state(L, u, ora, x, ora["history"][-2][1], tag="ph") > 0:
            continue
        sels = pipeline.select_per_head(q[u], ora["cmean"].astype(np.float32).astype(np.float64), ora["csize"],
                                        ora["offsets"], ora["k_clu_bits"], budget)
        if all(np.array_equal(sp[u * G + g], sels[g]["positions"]) for g in range(G)):
            ref = pipeline.decode_per_head(q[u], k[u], v[u], ora["k_clu_bits"], ora["v_clu_bits"],
                                           [x_["positions"] for x_ in sels], 16, n, n)
            err = np.abs(og[u] - ref).max()
            say(f"  unit {u}: per-head decode max abs err {err:.3g}")
            assert err <= DECODE_ATOL


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("G,n_sink,recent,budget,K", [
    (4, 16, 0, 1024, 48),
    (4, 16, 37, 2048, 48),
    (1, 16, 5, 256, 24),
    (16, 16, 300, 2048, 41),
    (8, 16, 20, 1024, 40),
    (13, 16, 1, 16, 40),      # G not a power of two, the 16-head tier; one chunk per unit
    (2, 0, 3, 64, 30),
    (4, 16, 11, 0, 20),
    (3, 16, 0, 500, 33),
    (4, 16, 2, 5000, 48),     # budget > m: full attention over every token
])
def test_decode_teacher_forced(G, n_sink, recent, budget, K):
    say(f"case: decode G={G} n_sink={n_sink} recent={recent} budget={budget} K={K}")
    units, nc = 3, n_sink + 4000
    n_total = nc + recent
    cap = n_total + 8
    ks, vs, cs = [], [], []
    for u in range(units):
        kb, vb, c = synth.make_unit_inputs(77, u, n_total, 64, capacity=cap)
        ks.append(kb), vs.append(vb), cs.append(c)
    k, v, cen = np.stack(ks), np.stack(vs), np.stack(cs)
    init = synth.make_init_indices(78, units, nc - n_sink, K)
    states = [pipeline.prefill_unit(k[u], nc, init[u], K, 2, n_sink=n_sink, v_bits=v[u])
              for u in range(units)]
    q = synth.make_queries(79, cen, G)
    L = gpu_layer(k, v, G, K, n_sink=n_sink, max_budget=max(budget, 1))
    load_state(L, states, n_sink=n_sink)
    L.set_counters(n_total, nc)
    sel_pos = np.zeros((units, max(budget, 1)), np.int32)
    cnt = np.zeros(units, np.int32)
    sels = []
    for u in range(units):
        sel = pipeline.select_unit(q[u], states[u]["cmean"], states[u]["csize"], states[u]["offsets"],
                                   states[u]["k_clu_bits"], budget)
        sels.append(sel)
        c = len(sel["positions"])
        sel_pos[u, :c] = sel["positions"]
        cnt[u] = c
    out = torch.zeros((units, G, D), dtype=torch.float32, device="cuda")
    L.sparse_decode(dev_bf16(q), to_dev(sel_pos, torch.int32), to_dev(cnt, torch.int32), budget, out)
    torch.cuda.synchronize()
    og = out.cpu().numpy()
    for u in range(units):
        ref = pipeline.decode_unit(q[u], k[u], v[u], states[u]["k_clu_bits"], states[u]["v_clu_bits"],
                                   sels[u]["positions"], n_sink, nc, n_total)
        err = np.abs(og[u] - ref).max()
        say(f"  unit {u}: max abs err {err:.3g}")
        assert err <= DECODE_ATOL


# ------------------------------------------------------------------ incremental


def test_incremental_teacher_forced():
    cfg = synth.CONFIGS["llama8b-incremental-b16"]
    say(f"case: incremental {cfg.name}, units 0-1")
    units = [0, 1]
    cap = cfg.n_tokens + cfg.new_tokens + 4
    k, v, cen = synth.make_layer_inputs(cfg, units=units, capacity=cap)
    init = synth.make_init_indices(cfg.init_seed, len(units), cfg.m, cfg.n_clusters)
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, 3, v_bits=v[u])
              for u in range(len(units))]
    kn, vn, newc = synth.make_new_tokens(cfg.data_seed, cen, cfg.new_tokens, cfg.new_components,
                                         cfg.new_fraction)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    load_state(L, states)
    L.set_counters(cfg.n_tokens, cfg.n_tokens)
    kd, vd = dev_bf16(kn), dev_bf16(vn)
    for i in range(cfg.new_tokens):
        L.append(kd[:, i].contiguous(), vd[:, i].contiguous())
    assert L.n_total == cfg.n_tokens + cfg.new_tokens
    L.incremental()
    assert L.n_clustered == L.n_total
    cen_all = np.concatenate([cen, newc], axis=1)
    q = synth.make_queries(cfg.query_seed, cen_all, cfg.group)
    qd = dev_bf16(q)
    sel_pos = torch.zeros((len(units), cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((len(units),), dtype=torch.int32, device="cuda")
    out = torch.zeros((len(units), cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    n_new = cfg.n_tokens + cfg.new_tokens
    compared = 0
    for u in range(len(units)):
        kf = k[u].copy()
        vf = v[u].copy()
        kf[cfg.n_tokens:n_new] = kn[u]
        vf[cfg.n_tokens:n_new] = vn[u]
        assert np.array_equal(host_bits(L.k_tok[u, :n_new]), kf[:n_new])
        ora = pipeline.incremental_unit(states[u], kf, n_new, v_bits=vf)
        x_new = bf16.widen(kn[u])
        a_g = L.assign[u, cfg.m:cfg.m + cfg.new_tokens].cpu().numpy()
        mism, unexc = compare_assign(a_g, ora["new_assign"], x_new, states[u]["cdir"])
        say(f"  unit {u}: new-token label mismatches {mism} (unexcused {unexc})")
        assert unexc == 0
        if mism:
            continue
        x_all = bf16.widen(kf[16:n_new])
        assert check_state(L, u, ora, x_all, states[u]["cdir"], tag="incr") == 0
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], kf, vf, ora, sp[u], cn[u], sel, diff, 16, n_new, n_new,
                                 tag=f"unit {u}:")
    assert compared >= 1, "no sampled unit's decode was compared"


def test_incremental_noop():
    say("case: incremental with no recent tokens")
    cfg = synth.CONFIGS["single-head-2k"]
    k, v, _ = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, 1, cfg.m, cfg.n_clusters)
    L = gpu_layer(k, v, 1, cfg.n_clusters)
    L.prefill(cfg.n_tokens, 3, to_dev(init, torch.int32))
    torch.cuda.synchronize()
    before = [t.clone() for t in (L.cdir, L.csum, L.offsets, L.perm, L.k_clu)]
    L.incremental()
    torch.cuda.synchronize()
    after = (L.cdir, L.csum, L.offsets, L.perm, L.k_clu)
    for a, b in zip(before, after):
        assert torch.equal(a, b)


def test_incremental_async_matches_sync():
    cfg = synth.CONFIGS["llama8b-incremental-b16"]
    units = [0, 1, 2, 3]
    say(f"case: async incremental + commit against the synchronous call ({cfg.name}, units 0-3, "
        f"+{cfg.new_tokens} keys)")
    cap = cfg.n_tokens + cfg.new_tokens + 4
    k, v, cen = synth.make_layer_inputs(cfg, units=units, capacity=cap)
    init = to_dev(synth.make_init_indices(cfg.init_seed, len(units), cfg.m, cfg.n_clusters), torch.int32)
    kn, vn, newc = synth.make_new_tokens(cfg.data_seed, cen, cfg.new_tokens, cfg.new_components,
                                         cfg.new_fraction)
    q = dev_bf16(synth.make_queries(cfg.query_seed, np.concatenate([cen, newc], axis=1), cfg.group))
    n_new = cfg.n_tokens + cfg.new_tokens
    layers = []
    for _ in range(2):
        L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
        L.prefill(cfg.n_tokens, 2, init)
        L.k_tok[:, cfg.n_tokens:n_new].copy_(dev_bf16(kn))
        L.v_tok[:, cfg.n_tokens:n_new].copy_(dev_bf16(vn))
        L.set_counters(n_new, cfg.n_tokens)
        layers.append(L)
    A, B = layers
    A.incremental()
    U = len(units)

    def recall_decode(L):
        sp = torch.full((U, cfg.budget), -1, dtype=torch.int32, device="cuda")
        cn = torch.zeros((U,), dtype=torch.int32, device="cuda")
        out = torch.zeros((U, cfg.group, D), dtype=torch.float32, device="cuda")
        L.select(q, cfg.budget, sp, cn)
        L.sparse_decode(q, sp, cn, cfg.budget, out)
        return sp, cn, out

    before = recall_decode(B)
    cur_before = [t.clone() for t in (B.offsets, B.cmean, B.k_clu, B.v_clu)]
    main = torch.cuda.current_stream()
    bg = torch.cuda.Stream()
    bg.wait_stream(main)
    with torch.cuda.stream(bg):
        B.incremental_async()
        done = torch.cuda.Event()
        done.record(bg)
    during = recall_decode(B)             # main stream, old state, beside the clustering
    main.wait_event(done)
    torch.cuda.synchronize()
    assert B.n_pending == n_new and B.n_clustered == cfg.n_tokens
    for a, b in zip(before, during):
        assert torch.equal(a, b), "recall / decode changed while the clustering ran"
    for a, b in zip(cur_before, (B.offsets, B.cmean, B.k_clu, B.v_clu)):
        assert torch.equal(a, b), "the current state changed before the commit"
    B.commit()
    assert B.n_pending == 0 and B.n_clustered == A.n_clustered == n_new
    m = n_new - 16
    for name in ("offsets", "cmean", "csum", "msum", "csize", "cdir"):
        assert torch.equal(getattr(A, name), getattr(B, name)), name
    for name in ("k_clu", "v_clu", "assign", "perm"):
        assert torch.equal(getattr(A, name)[:, :m], getattr(B, name)[:, :m]), name
    after = recall_decode(B)
    for a, b in zip(recall_decode(A), after):
        assert torch.equal(a, b)
    # the committed state and the recall / decode after the commit against the oracle
    sp, cn, og = (t.cpu().numpy() for t in after)
    init_h = init.cpu().numpy()
    qh = synth.make_queries(cfg.query_seed, np.concatenate([cen, newc], axis=1), cfg.group)
    compared = 0
    for u in (0, 3):
        kf, vf = k[u].copy(), v[u].copy()
        kf[cfg.n_tokens:n_new] = kn[u]
        vf[cfg.n_tokens:n_new] = vn[u]
        st = pipeline.prefill_unit(kf, cfg.n_tokens, init_h[u], cfg.n_clusters, 2, v_bits=vf)
        a_pre = B.assign[u, :cfg.m].cpu().numpy()
        if not np.array_equal(a_pre, st["assign"]):
            say(f"  async unit {u}: prefill labels differ in {int((a_pre != st['assign']).sum())} keys; skipped")
            continue
        ora = pipeline.incremental_unit(st, kf, n_new, v_bits=vf)
        x_all = bf16.widen(kf[16:n_new])
        if check_state(B, u, ora, x_all, st["cdir"], tag="async") > 0:
            continue
        sel = pipeline.select_unit(qh[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(B, u, sp, cn, ora, sel, cfg.budget)
        compared += check_decode(og[u], qh[u], kf, vf, ora, sp[u], cn[u], sel, diff, 16, n_new, n_new,
                                 tag=f"async unit {u}:")
    assert compared >= 1, "no sampled unit's decode was compared"


def test_append_select_matches_separate_calls():
    say("case: fused append + select against ckv_append then ckv_select (llama layer, 8 units)")
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    cap = cfg.n_tokens + 4
    k, v, cen = synth.make_layer_inputs(cfg, capacity=cap)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    q = dev_bf16(synth.make_queries(cfg.query_seed, cen, cfg.group))
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, 2, to_dev(init, torch.int32))
    kn, vn, _ = synth.make_new_tokens(cfg.data_seed, cen, 1, 0, 0.0)
    kd, vd = dev_bf16(kn[:, 0]), dev_bf16(vn[:, 0])
    outs = []
    for fused in (False, True):
        L.set_counters(cfg.n_tokens, cfg.n_tokens)
        L.k_tok[:, cfg.n_tokens].zero_()
        L.v_tok[:, cfg.n_tokens].zero_()
        sel_pos = torch.full((cfg.units, cfg.budget), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
        if fused:
            L.append_select(kd, vd, q, cfg.budget, sel_pos, cnt)
        else:
            L.append(kd, vd)
            L.select(q, cfg.budget, sel_pos, cnt)
        torch.cuda.synchronize()
        assert L.n_total == cfg.n_tokens + 1
        outs.append((sel_pos.clone(), cnt.clone(), L.k_tok[:, cfg.n_tokens].clone(), L.v_tok[:, cfg.n_tokens].clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert torch.equal(outs[1][2], kd) and torch.equal(outs[1][3], vd)


# ------------------------------------------------------------------ edge cases


@pytest.mark.parametrize("K,T", [(1, 3), (40, 5)])
def test_edge_zero_and_duplicate_keys(K, T):
    say(f"case: zero / duplicate keys K={K} T={T}")
    n = 16 + 700 + 7
    kb, vb, cen = synth.make_unit_inputs(91, 0, n, 8)
    kb[40:60] = 0                        # zero keys: score 0 everywhere, label 0
    kb[100:140] = kb[99]                 # duplicates of one key
    rng = np.random.default_rng(5)
    init = rng.choice(n - 16, K, replace=False).astype(np.int32)
    if K > 3:
        init[1] = 100 - 16                   # identical init directions -> empty clusters
        init[2] = 101 - 16
        init[3] = 45 - 16                    # a zero key as init -> zero direction
    ora = pipeline.prefill_unit(kb, n, init, K, T, v_bits=vb, history=True)
    L = gpu_layer(kb[None], vb[None], 1, K)
    L.prefill(n, T, to_dev(init[None], torch.int32))
    torch.cuda.synchronize()
    x = bf16.widen(kb[16:n])
    assert check_state(L, 0, ora, x, ora["history"][-2][1], tag="edge") == 0
    if K > 3:
        assert np.count_nonzero(ora["csize"] == 0) >= 1
    q = synth.make_queries(92, cen[None], 1)
    compared = 0
    for budget in (0, 50, 723, 800):
        sel_pos = torch.zeros((1, max(budget, 1)), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((1,), dtype=torch.int32, device="cuda")
        L.select(dev_bf16(q), budget, sel_pos, cnt)
        # the fused launch recalls the same positions and attends to them
        sp2, cn2 = torch.full_like(sel_pos, -1), torch.zeros_like(cnt)
        out2 = torch.zeros((1, 1, D), dtype=torch.float32, device="cuda")
        L.select_decode(dev_bf16(q), budget, sp2, cn2, out2)
        torch.cuda.synchronize()
        c = int(cnt[0])
        assert torch.equal(cn2, cnt) and torch.equal(sp2[:, :c], sel_pos[:, :c]), "fused recall differs"
        sel = pipeline.select_unit(q[0], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], budget)
        diff = compare_selection(L, 0, sel_pos.cpu().numpy(), cnt.cpu().numpy(), ora, sel, budget)
        compared += check_decode(out2.cpu().numpy()[0], q[0], kb, vb, ora, sel_pos.cpu().numpy()[0], c, sel, diff,
                                 16, n, n, tag=f"edge fused, budget {budget}")
    assert compared >= 1


@pytest.mark.parametrize("n_sink", [0, 16])
def test_edge_every_key_its_own_cluster(n_sink):
    # K = m: every clustered key starts as its own direction; with no sinks, token 0 is clustered too
    m = 300
    n = n_sink + m
    K, T, G = m, 2, 2
    say(f"case: K = m = {m}, n_sink = {n_sink}, {T} rounds, recall + decode")
    kb, vb, cen = synth.make_unit_inputs(141, 0, n, 24)
    init = np.arange(m, dtype=np.int32)
    ora = pipeline.prefill_unit(kb, n, init, K, T, n_sink=n_sink, v_bits=vb, history=True)
    L = gpu_layer(kb[None], vb[None], G, K, n_sink=n_sink)
    L.prefill(n, T, to_dev(init[None], torch.int32))
    torch.cuda.synchronize()
    x = bf16.widen(kb[n_sink:n])
    assert check_state(L, 0, ora, x, ora["history"][-2][1], n_sink=n_sink, tag="K=m") == 0
    q = synth.make_queries(142, cen[None], G)
    compared = 0
    for budget in (1, 37, m):
        sel_pos = torch.zeros((1, budget), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((1,), dtype=torch.int32, device="cuda")
        out = torch.zeros((1, G, D), dtype=torch.float32, device="cuda")
        L.select(dev_bf16(q), budget, sel_pos, cnt)
        L.sparse_decode(dev_bf16(q), sel_pos, cnt, budget, out)
        sp2, cn2, out2 = torch.full_like(sel_pos, -1), torch.zeros_like(cnt), torch.zeros_like(out)
        L.select_decode(dev_bf16(q), budget, sp2, cn2, out2)
        torch.cuda.synchronize()
        c = int(cnt[0])
        assert torch.equal(cn2, cnt) and torch.equal(sp2[:, :c], sel_pos[:, :c]), "fused recall differs"
        sel = pipeline.select_unit(q[0], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], budget)
        diff = compare_selection(L, 0, sel_pos.cpu().numpy(), cnt.cpu().numpy(), ora, sel, budget)
        for o, form in ((out, "two launches"), (out2, "fused")):
            compared += check_decode(o.cpu().numpy()[0], q[0], kb, vb, ora, sel_pos.cpu().numpy()[0], c, sel, diff,
                                     n_sink, n, n, tag=f"K=m {form}, budget {budget}")
    assert compared >= 2


def test_determinism():
    say("case: bitwise determinism of prefill, select, decode")
    cfg = synth.CONFIGS["single-head-2k"]
    k, v, cen = synth.make_layer_inputs(cfg)
    init = to_dev(synth.make_init_indices(cfg.init_seed, 1, cfg.m, cfg.n_clusters), torch.int32)
    q = dev_bf16(synth.make_queries(cfg.query_seed, cen, 4))
    outs = []
    for _ in range(2):
        L = gpu_layer(k, v, 4, cfg.n_clusters)
        L.prefill(cfg.n_tokens, cfg.iters, init)
        sel_pos = torch.zeros((1, cfg.budget), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((1,), dtype=torch.int32, device="cuda")
        out = torch.zeros((1, 4, D), dtype=torch.float32, device="cuda")
        L.select(q, cfg.budget, sel_pos, cnt)
        L.sparse_decode(q, sel_pos, cnt, cfg.budget, out)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (L.assign, L.cdir, L.csum, L.cmean, L.perm, L.k_clu, sel_pos, out)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ full size


def test_llama_stack_layer_full_size_sampled():
    cfg = synth.CONFIGS["llama8b-stack-32k-b8"]
    say(f"case: one full-size layer of {cfg.name} ({cfg.units} units), sampled units 5, 42")
    k, v, cen = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    del v
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    qd = dev_bf16(q)
    sel_pos = torch.zeros((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((cfg.units, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    assert np.all(cnt.cpu().numpy() == cfg.budget)
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in (5, 42, 61):
        _, vu, _ = synth.make_unit_inputs(cfg.data_seed, u, cfg.n_tokens, cfg.components)
        ora = pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=vu,
                                    history=True)
        x = bf16.widen(k[u][16:cfg.n_tokens])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], tag="full")
        if mism > MISMATCH_FRACTION * cfg.m:
            pytest.fail("too many label mismatches")
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], k[u], vu, ora, sp[u], cn[u], sel, diff, 16, cfg.n_tokens,
                                 cfg.n_tokens, tag=f"unit {u}:")
    assert compared >= 1, "no sampled unit's decode was compared"


def test_glm4_stack_layer_full_size_sampled():
    cfg = synth.CONFIGS["glm4-stack-32k-b16"]
    n_all = cfg.n_tokens + cfg.n_recent
    say(f"case: one full-size layer of {cfg.name} ({cfg.units} units, G={cfg.group}, K={cfg.n_clusters}, "
        f"{cfg.n_recent} recent), sampled units 3, 29")
    k, v, cen = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    L.set_counters(n_all, cfg.n_tokens)
    qd = dev_bf16(q)
    sel_pos = torch.zeros((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((cfg.units, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    assert np.all(cnt.cpu().numpy() == cfg.budget)
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in (3, 29, 17):
        ora = pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=v[u],
                                    history=True)
        x = bf16.widen(k[u][16:cfg.n_tokens])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], tag="full")
        if mism > MISMATCH_FRACTION * cfg.m:
            pytest.fail("too many label mismatches")
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, sp[u], cn[u], sel, diff, 16, cfg.n_tokens,
                                 n_all, tag=f"unit {u}:")
    assert compared >= 1, "no sampled unit's decode was compared"


def test_incremental_full_size_sampled():
    cfg = synth.CONFIGS["llama8b-incremental-b16"]
    n_new = cfg.n_tokens + cfg.new_tokens
    say(f"case: {cfg.name} at full size ({cfg.units} units): prefill, +{cfg.new_tokens} keys, incremental, "
        f"recall, decode; sampled units 7, 100")
    k, v, cen = synth.make_layer_inputs(cfg, capacity=n_new)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    kn, vn, newc = synth.make_new_tokens(cfg.data_seed, cen, cfg.new_tokens, cfg.new_components,
                                         cfg.new_fraction)
    k[:, cfg.n_tokens:n_new] = kn
    v[:, cfg.n_tokens:n_new] = vn
    q = synth.make_queries(cfg.query_seed, np.concatenate([cen, newc], axis=1), cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    L.set_counters(n_new, cfg.n_tokens)
    L.incremental()
    qd = dev_bf16(q)
    sel_pos = torch.zeros((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((cfg.units, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    assert L.n_clustered == n_new and np.all(cnt.cpu().numpy() == cfg.budget)
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in (7, 100):
        st = pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=v[u],
                                   history=True)
        a_pre = L.assign[u, :cfg.m].cpu().numpy()
        if not np.array_equal(a_pre, st["assign"]):
            # a near-tie decided differently in the prefill: the bar for that is the prefill test's;
            # the incremental comparison needs equal starting states
            say(f"  unit {u}: prefill labels differ in {int((a_pre != st['assign']).sum())} keys; skipped")
            continue
        ora = pipeline.incremental_unit(st, k[u], n_new, v_bits=v[u])
        x_all = bf16.widen(k[u][16:n_new])
        if check_state(L, u, ora, x_all, st["cdir"], tag="incr-full") > 0:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, sp, cn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, sp[u], cn[u], sel, diff, 16, n_new, n_new,
                                 tag=f"unit {u}:")
    assert compared >= 1, "no sampled unit's decode was compared"


# ------------------------------------------------------------------ drift split


def _reserve_init(cfg, units, reserve):
    init = synth.make_init_indices(cfg.init_seed, units, cfg.m, cfg.n_clusters)
    return np.concatenate([init, np.full((units, reserve), -1, np.int32)], axis=1)


def _split_threshold(states, q):
    """A threshold halfway between two neighbouring drifts (near quantile ``q`` of
    unit 0's clusters with >= 2 members), checked against every unit: no drift
    lies within 1e-12 of it, and no two candidate drifts are within 1e-12 (so the
    pairing order cannot hinge on summation order)."""
    from oracle import kmeans
    d0 = kmeans.drift(states[0]["csum"], states[0]["csize"])
    d = np.sort(d0[states[0]["csize"] >= 2])
    i = int(q * (len(d) - 1))
    tau = 0.5 * (d[i] + d[i + 1])
    for st in states:
        dr = kmeans.drift(st["csum"], st["csize"])[st["csize"] >= 2]
        assert np.min(np.abs(dr - tau)) > 1e-12
        c = np.sort(dr[dr > tau])
        assert len(c) < 2 or np.min(np.diff(c)) > 1e-12
    return float(tau)


def _check_split(L, states, k, v, tau, tag):
    oras = [pipeline.split_unit(st, k[u], tau, v_bits=v[u]) for u, st in enumerate(states)]
    L.split(tau)
    torch.cuda.synchronize()
    total_pairs = 0
    for u, ora in enumerate(oras):
        m = len(ora["assign"])
        total_pairs += len(ora["pairs"])
        a_g = L.assign[u, :m].cpu().numpy()
        say(f"  {tag} unit {u}: {len(ora['pairs'])} splits, labels differing {int(np.sum(a_g != ora['assign']))}")
        assert np.array_equal(a_g, ora["assign"]), "split labels differ"
        x = bf16.widen(k[u][16:ora["n_clustered"]])
        assert check_state(L, u, ora, x, ora["cdir"], tag=tag) == 0
    return oras, total_pairs


def test_split_after_prefill_with_reserved_slots():
    cfg = synth.CONFIGS["single-head-2k"]
    say("case: drift split, teacher-forced prefill state with 8 reserved slots, 3 units")
    U, R = 3, 8
    k, v, _ = synth.make_layer_inputs(cfg, units=list(range(U)))
    init = _reserve_init(cfg, U, R)
    K = cfg.n_clusters + R
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], K, cfg.iters, v_bits=v[u]) for u in range(U)]
    for st in states:
        assert np.all(st["csize"][cfg.n_clusters:] == 0)
    for q in (0.5, 0.9):
        L = gpu_layer(k, v, 1, K)
        load_state(L, states)
        L.set_counters(cfg.n_tokens, cfg.n_tokens)
        _, pairs = _check_split(L, states, k, v, _split_threshold(states, q), f"q={q}")
        assert pairs > 0


def test_split_on_gpu_prefill_with_reserved_slots():
    cfg = synth.CONFIGS["single-head-2k"]
    say("case: GPU prefill with 8 reserved slots, then drift split, 3 units")
    U, R = 3, 8
    k, v, _ = synth.make_layer_inputs(cfg, units=list(range(U)))
    init = _reserve_init(cfg, U, R)
    K = cfg.n_clusters + R
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], K, cfg.iters, v_bits=v[u]) for u in range(U)]
    L = gpu_layer(k, v, 1, K)
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    torch.cuda.synchronize()
    for u in range(U):
        x = bf16.widen(k[u][16:cfg.n_tokens])
        assert check_state(L, u, states[u], x, states[u]["cdir"], tag="prefill") == 0
    _check_split(L, states, k, v, _split_threshold(states, 0.5), "split")


def test_split_without_free_slot_only_rebuilds():
    cfg = synth.CONFIGS["single-head-2k"]
    say("case: drift split with no empty slot (every cluster a candidate)")
    k, v, _ = synth.make_layer_inputs(cfg, units=[0, 1])
    init = synth.make_init_indices(cfg.init_seed, 2, cfg.m, cfg.n_clusters)
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=v[u])
              for u in range(2)]
    assert all(np.all(st["csize"] > 0) for st in states)
    L = gpu_layer(k, v, 1, cfg.n_clusters)
    load_state(L, states)
    L.set_counters(cfg.n_tokens, cfg.n_tokens)
    _, pairs = _check_split(L, states, k, v, -1.0, "no-slot")
    assert pairs == 0


def test_split_more_pairs_than_workgroups_without_sinks():
    """Every cluster with two or more members splits (threshold -1), 40 reserved
    slots: more pairs per unit than the move kernel's 16 workgroups, so some
    take two pairs; no sinks (token 0 is clustered too)."""
    cfg = synth.CONFIGS["single-head-2k"]
    U, R, n_sink = 2, 40, 0
    say(f"case: drift split of every cluster, {R} reserved slots, n_sink = 0, {U} units")
    from oracle import kmeans
    k, v, _ = synth.make_layer_inputs(cfg, units=list(range(U)))
    m = cfg.n_tokens - n_sink
    init = np.concatenate([synth.make_init_indices(cfg.init_seed, U, m, cfg.n_clusters),
                           np.full((U, R), -1, np.int32)], axis=1)
    K = cfg.n_clusters + R
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], K, cfg.iters, n_sink=n_sink, v_bits=v[u])
              for u in range(U)]
    for st in states:   # the pairing order must not hinge on summation order
        dr = np.sort(kmeans.drift(st["csum"], st["csize"])[st["csize"] >= 2])
        assert len(dr) > 16 and np.min(np.diff(dr)) > 1e-12
    oras = [pipeline.split_unit(st, k[u], -1.0, n_sink=n_sink, v_bits=v[u]) for u, st in enumerate(states)]
    L = gpu_layer(k, v, 1, K, n_sink=n_sink)
    load_state(L, states, n_sink=n_sink)
    L.set_counters(cfg.n_tokens, cfg.n_tokens)
    L.split(-1.0)
    torch.cuda.synchronize()
    for u, ora in enumerate(oras):
        assert len(ora["pairs"]) > 16
        a_g = L.assign[u, :m].cpu().numpy()
        say(f"  unit {u}: {len(ora['pairs'])} splits, labels differing {int(np.sum(a_g != ora['assign']))}")
        assert np.array_equal(a_g, ora["assign"]), "split labels differ"
        x = bf16.widen(k[u][n_sink:cfg.n_tokens])
        assert check_state(L, u, ora, x, ora["cdir"], n_sink=n_sink, tag="split-all") == 0


def test_split_many_clusters():
    """700 slots (600 clusters of about 3 keys plus 100 reserved): the plan kernel's
    size, free-slot and ranking passes cover more clusters than its 256 threads."""
    cfg = synth.CONFIGS["single-head-2k"]
    U, R, K0 = 2, 100, 600
    say(f"case: drift split with {K0} clusters + {R} reserved slots, {U} units")
    k, v, _ = synth.make_layer_inputs(cfg, units=list(range(U)))
    init = np.concatenate([synth.make_init_indices(cfg.init_seed, U, cfg.m, K0),
                           np.full((U, R), -1, np.int32)], axis=1)
    K = K0 + R
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], K, 3, v_bits=v[u]) for u in range(U)]
    L = gpu_layer(k, v, 1, K)
    load_state(L, states)
    L.set_counters(cfg.n_tokens, cfg.n_tokens)
    _, pairs = _check_split(L, states, k, v, _split_threshold(states, 0.5), "split-700")
    assert pairs == U * R


def test_split_after_incremental_new_components_then_recall_and_decode():
    cfg = synth.CONFIGS["llama8b-incremental-b16"]
    U, R = 2, 16
    say(f"case: drift split after +{cfg.new_tokens} keys from {cfg.new_components} new components, "
        f"Llama layer shape, K = {cfg.n_clusters} + {R} reserved, units 0-1, then recall and decode")
    n_new = cfg.n_tokens + cfg.new_tokens
    k, v, cen = synth.make_layer_inputs(cfg, units=list(range(U)), capacity=n_new + 4)
    init = _reserve_init(cfg, U, R)
    K = cfg.n_clusters + R
    states = [pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], K, 3, v_bits=v[u]) for u in range(U)]
    kn, vn, newc = synth.make_new_tokens(cfg.data_seed, cen, cfg.new_tokens, cfg.new_components,
                                         cfg.new_fraction)
    k[:, cfg.n_tokens:n_new] = kn
    v[:, cfg.n_tokens:n_new] = vn
    states = [pipeline.incremental_unit(states[u], k[u], n_new, v_bits=v[u]) for u in range(U)]
    L = gpu_layer(k, v, cfg.group, K, max_budget=cfg.budget)
    load_state(L, states)
    L.set_counters(n_new, n_new)
    oras, pairs = _check_split(L, states, k, v, _split_threshold(states, 0.5), "split")
    assert pairs == U * R                       # more candidates than reserved slots
    q = synth.make_queries(cfg.query_seed, np.concatenate([cen, newc], axis=1), cfg.group)
    qd = dev_bf16(q)
    sel_pos = torch.zeros((U, cfg.budget), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((U,), dtype=torch.int32, device="cuda")
    out = torch.zeros((U, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select(qd, cfg.budget, sel_pos, cnt)
    L.sparse_decode(qd, sel_pos, cnt, cfg.budget, out)
    torch.cuda.synchronize()
    sp, cn, og = sel_pos.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy()
    for u, ora in enumerate(oras):
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        if compare_selection(L, u, sp, cn, ora, sel, cfg.budget) == 0:
            ref = pipeline.decode_unit(q[u], k[u], v[u], ora["k_clu_bits"], ora["v_clu_bits"], sel["positions"],
                                       16, n_new, n_new)
            err = np.abs(og[u] - ref).max()
            say(f"  unit {u}: decode max abs err {err:.3g}")
            assert err <= DECODE_ATOL


# ------------------------------------------------------------------ HIP graphs


@pytest.mark.parametrize("append", [False, True])
def test_graph_replay_matches_eager(append):
    """Recall + decode (or the bench's step: fused append + recall, then decode)
    captured once in a HIP graph and replayed three times, with other eager
    recall / decode work and torch work between the replays: every replay's
    positions, counts and outputs equal the eager call's bit for bit."""
    U, G, K, m, r, budget = 6, 4, 48, 4000, 9, 512
    n = 16 + m
    say(f"case: graph replay of {'append + ' if append else ''}recall + decode, {U} units, G = {G}, "
        f"K = {K}, m = {m}, {r} recent rows")
    parts = [synth.make_unit_inputs(7100, u, n + r, 32, capacity=n + r + 1) for u in range(U)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(7200, U, m, K)
    L = gpu_layer(k, v, G, K, max_budget=budget)
    L.prefill(n, 3, to_dev(init, torch.int32))
    L.set_counters(n + r, n)
    q0 = dev_bf16(synth.make_queries(7300, cen, G))
    q1 = dev_bf16(synth.make_queries(7301, cen, G))
    new_rows = synth.make_unit_inputs(7400, 0, U, 32)
    k_new, v_new = dev_bf16(new_rows[0]), dev_bf16(new_rows[1])

    def buffers():
        return (torch.zeros((U, budget), dtype=torch.int32, device="cuda"),
                torch.zeros((U,), dtype=torch.int32, device="cuda"),
                torch.zeros((U, G, D), dtype=torch.float32, device="cuda"))

    def run(q, bufs, with_append=False):
        if with_append:   # the decoded token's row n + r, then n_total = n + r + 1
            L.append_select(k_new, v_new, q, budget, bufs[0], bufs[1])
        else:
            L.select(q, budget, bufs[0], bufs[1])
        L.sparse_decode(q, bufs[0], bufs[1], budget, bufs[2])

    eager, other, static = buffers(), buffers(), buffers()
    run(q0, eager, append)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    L.set_counters(n + r, n)
    with torch.cuda.stream(side):
        run(q0, static, append)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    L.set_counters(n + r, n)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(q0, static, append)
    torch.cuda.synchronize()
    for rep in range(3):
        run(q1, other)                      # eager work on the same layer and workspace
        _ = (other[2] * 2.0).sum()          # and some torch work
        for t in static:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}: positions equal {torch.equal(static[0], eager[0])}, "
            f"outputs equal {torch.equal(static[2], eager[2])}")
        assert torch.equal(static[1], eager[1])
        assert torch.equal(static[0], eager[0])
        assert torch.equal(static[2], eager[2])
    assert not torch.equal(other[2], eager[2])      # the other query really differs
