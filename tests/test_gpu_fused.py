"""GPU parity of the fused recall + decode launch (ckv_select_decode and its
append / per-query-head forms) against the float64 oracle.

The fused launch recalls each set in every one of its workgroups and streams
the rows from the cluster index; its recalled positions must be the oracle's
recall (same bar as ckv_select: equal unless the oracle's boundary has a
near-tie) and its output the oracle's attention over them (max abs error
<= 2e-3).  Where the fused and the separate calls run the same arithmetic (the
scores and the selection) their positions are also compared with each other.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import (MISMATCH_FRACTION, check_decode, check_state, compare_selection, dev_bf16, gpu_layer,
                      load_state, say, to_dev)
from oracle import bf16, pipeline

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

D = 128


def _bufs(sets, budget, units, G):
    return (torch.full((sets, max(budget, 1)), -1, dtype=torch.int32, device="cuda"),
            torch.zeros((sets,), dtype=torch.int32, device="cuda"),
            torch.zeros((units, G, D), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("G,n_sink,recent,budget,K,units", [
    (4, 16, 0, 1024, 48, 3),
    (4, 16, 37, 2048, 48, 3),
    (1, 16, 5, 256, 24, 3),
    (16, 16, 300, 2048, 41, 2),
    (8, 16, 20, 1024, 40, 3),
    (13, 16, 1, 16, 40, 3),
    (2, 0, 3, 64, 30, 3),
    (4, 16, 11, 0, 20, 3),
    (3, 16, 0, 500, 33, 3),
    (4, 16, 2, 5000, 48, 3),     # budget > m: every cluster, full attention
    (4, 16, 7, 1500, 48, 40),    # 40 sets: 7 chunks per set
    (4, 16, 7, 1500, 48, 300),   # more sets than CUs: one chunk per set
])
def test_fused_teacher_forced(G, n_sink, recent, budget, K, units):
    say(f"case: fused recall + decode, G={G} n_sink={n_sink} recent={recent} budget={budget} K={K} units={units}")
    nc = n_sink + 4000
    n_total = nc + recent
    cap = n_total + 8
    parts = [synth.make_unit_inputs(77, u, n_total, 64, capacity=cap) for u in range(units)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(78, units, nc - n_sink, K)
    checked = [u for u in range(units) if u < 3 or u == units - 1]
    states = {u: pipeline.prefill_unit(k[u], nc, init[u], K, 2, n_sink=n_sink, v_bits=v[u]) for u in checked}
    # the unchecked units get the first unit's state (only the checked units are compared)
    q = synth.make_queries(79, cen, G)
    L = gpu_layer(k, v, G, K, n_sink=n_sink, max_budget=max(budget, 1))
    load_state(L, [states.get(u, states[0]) for u in range(units)], n_sink=n_sink)
    L.set_counters(n_total, nc)
    qd = dev_bf16(q)
    sp, cn, out = _bufs(units, budget, units, G)
    L.select_decode(qd, budget, sp, cn, out)
    sp2, cn2, _ = _bufs(units, budget, units, G)
    L.select(qd, budget, sp2, cn2)
    torch.cuda.synchronize()
    m = nc - n_sink
    assert torch.equal(cn, cn2) and np.all(cn.cpu().numpy() == min(budget, m))
    c = min(budget, m)
    assert torch.equal(sp[:, :c], sp2[:, :c]), "fused recall differs from ckv_select"
    spn, cnn, og = sp.cpu().numpy(), cn.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in checked:
        st = states[u]
        sel = pipeline.select_unit(q[u], st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], budget)
        diff = compare_selection(L, u, spn, cnn, st, sel, budget)
        compared += check_decode(og[u], q[u], k[u], v[u], st, spn[u], cnn[u], sel, diff, n_sink, nc, n_total,
                                 tag=f"unit {u}: fused")
    assert compared >= 1, "no checked unit's decode was compared"


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
def test_fused_random_shapes_end_to_end(case):
    """Seeded random shapes through prefill and the fused recall + decode
    (with the appended token: the decoded token's row is written and attended)."""
    rng = np.random.default_rng(9500 + case)
    U, n_sink, K, m, G, T, budget, r, C = _random_case(rng)
    n = n_sink + m
    say(f"case {case}: units {U}, n_sink {n_sink}, K {K}, m {m}, G {G}, rounds {T}, budget {budget}, "
        f"recent {r} + 1 appended, components {C}")
    parts = [synth.make_unit_inputs(9600 + case, u, n + r + 1, C, capacity=n + r + 2) for u in range(U)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(9700 + case, U, m, K)
    q = synth.make_queries(9800 + case, cen, G)
    # the appended row arrives through k_new / v_new, not through k_tok
    k_new, v_new = k[:, n + r].copy(), v[:, n + r].copy()
    k_in, v_in = k.copy(), v.copy()
    k_in[:, n + r] = 0
    v_in[:, n + r] = 0
    L = gpu_layer(k_in, v_in, G, K, n_sink=n_sink, max_budget=max(budget, 1))
    L.prefill(n, T, to_dev(init, torch.int32))
    L.set_counters(n + r, n)
    qd = dev_bf16(q)
    sp, cn, out = _bufs(U, budget, U, G)
    L.append_select_decode(dev_bf16(k_new), dev_bf16(v_new), qd, budget, sp, cn, out)
    torch.cuda.synchronize()
    assert L.n_total == n + r + 1
    assert np.array_equal(L.k_tok[:, n + r].view(torch.int16).cpu().numpy().view(np.uint16), k_new)
    assert np.array_equal(L.v_tok[:, n + r].view(torch.int16).cpu().numpy().view(np.uint16), v_new)
    spn = sp.cpu().numpy()[:, :budget]
    cnn, og = cn.cpu().numpy(), out.cpu().numpy()
    total_mism = compared = 0
    for u in range(U):
        ora = pipeline.prefill_unit(k[u], n, init[u], K, T, n_sink=n_sink, v_bits=v[u], history=True)
        x = bf16.widen(k[u][n_sink:n])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], n_sink=n_sink, tag=f"case {case}")
        total_mism += mism
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], budget)
        diff = compare_selection(L, u, spn, cnn, ora, sel, budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, spn[u], cnn[u], sel, diff, n_sink, n, n + r + 1,
                                 tag=f"unit {u}:")
    assert total_mism <= max(1, MISMATCH_FRACTION * U * m)
    assert compared >= 1


def _fused_exact(L, st, q, k, v, budget, n_sink, nc, n_total, tag):
    """Fused call on unit 0 against the oracle where ties decide the recall:
    the token sets must be equal (the tie rules fix them), and the output too."""
    G = q.shape[1]
    sp, cn, out = _bufs(1, budget, 1, G)
    L.select_decode(dev_bf16(q), budget, sp, cn, out)
    sp2, cn2, _ = _bufs(1, budget, 1, G)
    L.select(dev_bf16(q), budget, sp2, cn2)
    torch.cuda.synchronize()
    m = nc - n_sink
    c = min(budget, m)
    assert int(cn[0]) == c and torch.equal(sp[:, :c], sp2[:, :c]), "fused recall differs from ckv_select"
    spn, cnn, og = sp.cpu().numpy(), cn.cpu().numpy(), out.cpu().numpy()
    sel = pipeline.select_unit(q[0], st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], budget)
    diff = compare_selection(L, 0, spn, cnn, st, sel, budget)
    assert diff == 0, f"{tag}: recall differs by {diff} tokens where only ties decide"
    assert check_decode(og[0], q[0], k[0], v[0], st, spn[0], cnn[0], sel, 0, n_sink, nc, n_total, tag=tag) == 1


def test_fused_degenerate_scores():
    """q = 0: every cluster and cut-token score is 0, so the score range is
    degenerate and both selections take their radix fallback; ties go to the
    smaller cluster index and the smaller position (earlier token)."""
    say("case: fused recall + decode with a zero query (all scores tie)")
    n_sink, K, recent = 16, 40, 9
    nc = n_sink + 3000
    n_total = nc + recent
    kb, vb, cen = synth.make_unit_inputs(81, 0, n_total, 24, capacity=n_total + 8)
    init = synth.make_init_indices(82, 1, nc - n_sink, K)[0]
    st = pipeline.prefill_unit(kb, nc, init, K, 2, n_sink=n_sink, v_bits=vb)
    L = gpu_layer(kb[None], vb[None], 2, K, n_sink=n_sink, max_budget=3100)
    load_state(L, [st], n_sink=n_sink)
    L.set_counters(n_total, nc)
    q = np.zeros((1, 2, D), np.uint16)
    for budget in (1, 77, 1500, 2999, 3100):
        _fused_exact(L, st, q, kb[None], vb[None], budget, n_sink, nc, n_total, tag=f"zero query, budget {budget}")


def test_fused_crowded_crossing_bucket():
    """100 clusters with one shared scoring centroid (so one shared score, in
    the middle of the range): the bucket where the budget is crossed holds more
    candidates than the exact in-bucket rank takes, and the selection falls
    back to the radix select; ties among the 100 go to the smaller index."""
    say("case: fused recall + decode with 100 equal cluster scores at the cut")
    n_sink, K, recent, G = 16, 200, 3, 4
    nc = n_sink + 8000
    n_total = nc + recent
    kb, vb, cen = synth.make_unit_inputs(83, 0, n_total, 96, capacity=n_total + 8)
    init = synth.make_init_indices(84, 1, nc - n_sink, K)[0]
    st = pipeline.prefill_unit(kb, nc, init, K, 2, n_sink=n_sink, v_bits=vb)
    q = synth.make_queries(85, cen[None], G)
    qbar = bf16.widen(q[0]).sum(axis=0)
    mu = st["cmean"].astype(np.float32).astype(np.float64)  # the GPU holds f32 centroids
    scores = mu @ qbar
    group = np.argsort(scores)[50:150]              # 100 clusters from the middle of the order
    common = mu[group].mean(axis=0).astype(np.float32).astype(np.float64)
    mu[group] = common
    st = dict(st, cmean=mu)
    scores = np.where(st["csize"] > 0, mu @ qbar, -np.inf)
    order = sorted(range(K), key=lambda j: (-scores[j], j))
    pos = [order.index(j) for j in group]
    first = min(pos)
    before = int(sum(st["csize"][order[i]] for i in range(first)))
    inside = int(sum(st["csize"][j] for j in group))
    L = gpu_layer(kb[None], vb[None], G, K, n_sink=n_sink, max_budget=8000)
    load_state(L, [st], n_sink=n_sink)
    L.set_counters(n_total, nc)
    for budget in (before + inside // 2, before + inside // 3 + 1, before + 1):
        _fused_exact(L, st, q, kb[None], vb[None], budget, n_sink, nc, n_total,
                     tag=f"crowded bucket, budget {budget}")


def test_fused_glm4_layer_full_size():
    """One full GLM4-shaped layer (32 units, G = 16, K = 410, 300 recent rows,
    budget 2048): 8 chunks per set in the fused launch."""
    cfg = synth.CONFIGS["glm4-stack-32k-b16"]
    n_all = cfg.n_tokens + cfg.n_recent
    say(f"case: fused recall + decode on a full {cfg.name} layer; sampled units 6, 25")
    k, v, cen = synth.make_layer_inputs(cfg)
    init = synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters)
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, to_dev(init, torch.int32))
    L.set_counters(n_all, cfg.n_tokens)
    qd = dev_bf16(q)
    sp, cn, out = _bufs(cfg.units, cfg.budget, cfg.units, cfg.group)
    L.select_decode(qd, cfg.budget, sp, cn, out)
    sp2, cn2, _ = _bufs(cfg.units, cfg.budget, cfg.units, cfg.group)
    L.select(qd, cfg.budget, sp2, cn2)
    torch.cuda.synchronize()
    assert torch.equal(sp, sp2) and torch.equal(cn, cn2)
    spn, cnn, og = sp.cpu().numpy(), cn.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in (6, 25):
        ora = pipeline.prefill_unit(k[u], cfg.n_tokens, init[u], cfg.n_clusters, cfg.iters, v_bits=v[u],
                                    history=True)
        x = bf16.widen(k[u][16:cfg.n_tokens])
        if check_state(L, u, ora, x, ora["history"][-2][1], tag="glm4 fused"):
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"],
                                   cfg.budget)
        diff = compare_selection(L, u, spn, cnn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, spn[u], cnn[u], sel, diff, 16, cfg.n_tokens, n_all,
                                 tag=f"unit {u}:")
    assert compared >= 1


def test_fused_append_matches_separate_calls():
    """ckv_append_select_decode against ckv_append + ckv_select + ckv_sparse_decode
    on the Llama layer shape: the same positions, outputs within float rounding
    of each other, the same cache rows afterwards."""
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    say(f"case: fused append + recall + decode against the separate calls ({cfg.name})")
    cap = cfg.n_tokens + 4
    k, v, cen = synth.make_layer_inputs(cfg, capacity=cap)
    init = to_dev(synth.make_init_indices(cfg.init_seed, cfg.units, cfg.m, cfg.n_clusters), torch.int32)
    q = dev_bf16(synth.make_queries(cfg.query_seed, cen, cfg.group))
    new = synth.make_unit_inputs(4242, 0, cfg.units, 16)
    k_new, v_new = dev_bf16(new[0]), dev_bf16(new[1])
    outs = []
    for fused in (True, False):
        L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
        L.prefill(cfg.n_tokens, 2, init)
        sp, cn, out = _bufs(cfg.units, cfg.budget, cfg.units, cfg.group)
        if fused:
            L.append_select_decode(k_new, v_new, q, cfg.budget, sp, cn, out)
        else:
            L.append(k_new, v_new)
            L.select(q, cfg.budget, sp, cn)
            L.sparse_decode(q, sp, cn, cfg.budget, out)
        torch.cuda.synchronize()
        assert L.n_total == cfg.n_tokens + 1
        outs.append((sp, cn, out, L.k_tok.clone(), L.v_tok.clone()))
    (a_sp, a_cn, a_out, a_k, a_v), (b_sp, b_cn, b_out, b_k, b_v) = outs
    assert torch.equal(a_sp, b_sp) and torch.equal(a_cn, b_cn)
    assert torch.equal(a_k, b_k) and torch.equal(a_v, b_v)
    err = float((a_out - b_out).abs().max())
    say(f"  fused vs separate output max abs difference {err:.3g}")
    assert err <= 1e-4


def test_fused_graph_replay_matches_eager():
    """The bench's fused step (append + recall + decode in one launch) captured
    once in a HIP graph and replayed three times, with other eager work on the
    same layer and workspace between replays: every replay equals the eager call."""
    U, G, K, m, r, budget = 6, 4, 48, 4000, 9, 512
    n = 16 + m
    say(f"case: graph replay of the fused append + recall + decode, {U} units")
    parts = [synth.make_unit_inputs(7100, u, n + r, 32, capacity=n + r + 1) for u in range(U)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(7200, U, m, K)
    L = gpu_layer(k, v, G, K, max_budget=budget)
    L.prefill(n, 3, to_dev(init, torch.int32))
    q0 = dev_bf16(synth.make_queries(7300, cen, G))
    q1 = dev_bf16(synth.make_queries(7301, cen, G))
    new_rows = synth.make_unit_inputs(7400, 0, U, 32)
    k_new, v_new = dev_bf16(new_rows[0]), dev_bf16(new_rows[1])
    eager, other, static = _bufs(U, budget, U, G), _bufs(U, budget, U, G), _bufs(U, budget, U, G)
    L.set_counters(n + r, n)
    L.append_select_decode(k_new, v_new, q0, budget, *eager)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    L.set_counters(n + r, n)
    with torch.cuda.stream(side):
        L.append_select_decode(k_new, v_new, q0, budget, *static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    L.set_counters(n + r, n)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.append_select_decode(k_new, v_new, q0, budget, *static)
    torch.cuda.synchronize()
    for rep in range(3):
        L.select_decode(q1, budget, *other)   # eager work on the same layer and workspace
        _ = (other[2] * 2.0).sum()
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
    assert not torch.equal(other[2], eager[2])


def test_fused_prefetch_hint_changes_nothing():
    """The next-layer hint only warms caches: with or without it (and with a
    layer of another shape, which is ignored) the fused call writes the same bits."""
    U, G, K, m, r, budget = 40, 4, 48, 4000, 5, 1000
    n = 16 + m
    say(f"case: fused call with and without the prefetch hint, {U} units")
    parts = [synth.make_unit_inputs(8100 + i, u, n + r, 32) for i in range(2) for u in range(U)]
    layers = []
    for i in range(2):
        k = np.stack([p[0] for p in parts[i * U:(i + 1) * U]])
        v = np.stack([p[1] for p in parts[i * U:(i + 1) * U]])
        L = gpu_layer(k, v, G, K, max_budget=budget)
        L.prefill(n, 2, to_dev(synth.make_init_indices(8200 + i, U, m, K), torch.int32))
        L.set_counters(n + r, n)
        layers.append(L)
    other = gpu_layer(np.stack([p[0] for p in parts[:3]]), np.stack([p[1] for p in parts[:3]]), G, K, max_budget=budget)
    cen = np.stack([p[2] for p in parts[:U]])
    q = dev_bf16(synth.make_queries(8300, cen, G))
    results = []
    for hint in (None, layers[1], other, layers[0]):
        sp, cn, out = _bufs(U, budget, U, G)
        layers[0].select_decode(q, budget, sp, cn, out, next_layer=hint)
        torch.cuda.synchronize()
        results.append((sp, cn, out))
    for sp, cn, out in results[1:]:
        assert torch.equal(sp, results[0][0]) and torch.equal(cn, results[0][1]) and torch.equal(out, results[0][2])
