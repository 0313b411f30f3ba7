"""The allocation-free fused call (ckv_select_decode_noalloc) against the
workspace form (ckv_select_decode) and the float64 oracle.

Three calls in a row share the library's per-device scratch: a 16-unit layer,
then a smaller one (3 units, a smaller budget, fewer chunks), then a layer
whose cut cluster holds 6000 tokens (its scores go through the scratch's cut
area).  Each must give exactly the workspace form's positions, counts and
outputs, and the oracle's recall and attention.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_decode, compare_selection, dev_bf16, gpu_layer, load_state, say
from oracle import pipeline

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

from semantic_cluster_sparse_amd import ckv  # noqa: E402

D = 128


def _bufs(units, budget, G):
    return (torch.full((units, max(budget, 1)), -1, dtype=torch.int32, device="cuda"),
            torch.zeros((units,), dtype=torch.int32, device="cuda"),
            torch.zeros((units, G, D), dtype=torch.float32, device="cuda"))


def _compare(L, q_bits, budget, G, states, k, v, nc, n_total, n_sink, tag):
    qd = dev_bf16(q_bits)
    units = q_bits.shape[0]
    a = _bufs(units, budget, G)
    b = _bufs(units, budget, G)
    L.select_decode(qd, budget, *a)
    L.select_decode_noalloc(qd, budget, *b)
    torch.cuda.synchronize()
    say(f"  {tag}: positions equal {torch.equal(a[0], b[0])}, counts equal {torch.equal(a[1], b[1])}, "
        f"outputs equal {torch.equal(a[2], b[2])}")
    assert torch.equal(a[1], b[1]) and torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])
    spn, cnn, og = b[0].cpu().numpy(), b[1].cpu().numpy(), b[2].cpu().numpy()
    compared = 0
    for u, st in states.items():
        sel = pipeline.select_unit(q_bits[u], st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], budget)
        diff = compare_selection(L, u, spn, cnn, st, sel, budget)
        compared += check_decode(og[u], q_bits[u], k[u], v[u], st, spn[u], cnn[u], sel, diff, n_sink, nc, n_total,
                                 tag=f"{tag} unit {u}:")
    assert compared >= 1


def _teacher_forced(units, K, m, G, recent, seed):
    n_sink = 16
    nc = n_sink + m
    n_total = nc + recent
    parts = [synth.make_unit_inputs(seed, u, n_total, 64, capacity=n_total + 4) for u in range(units)]
    k = np.stack([p[0] for p in parts])
    v = np.stack([p[1] for p in parts])
    cen = np.stack([p[2] for p in parts])
    init = synth.make_init_indices(seed + 1, units, m, K)
    states = {u: pipeline.prefill_unit(k[u], nc, init[u], K, 2, v_bits=v[u]) for u in range(units)}
    L = gpu_layer(k, v, G, K, max_budget=2048)
    load_state(L, [states[u] for u in range(units)])
    L.set_counters(n_total, nc)
    q = synth.make_queries(seed + 2, cen, G)
    return L, q, states, k, v, nc, n_total


def test_noalloc_matches_workspace_call_three_calls():
    assert ckv.ckv_select_decode_noalloc_limit() == 16 << 20
    say("case: no-alloc call 1 of 3: 16 units, K 48, m 4000, G 4, budget 1024, 7 recent rows")
    L, q, states, k, v, nc, nt = _teacher_forced(16, 48, 4000, 4, 7, 6100)
    _compare(L, q, 1024, 4, {0: states[0], 15: states[15]}, k, v, nc, nt, 16, "call 1")

    say("case: no-alloc call 2 of 3 (smaller): 3 units, K 20, m 1500, G 2, budget 200, 3 recent rows")
    L2, q2, states2, k2, v2, nc2, nt2 = _teacher_forced(3, 20, 1500, 2, 3, 6200)
    _compare(L2, q2, 200, 2, states2, k2, v2, nc2, nt2, 16, "call 2")

    say("case: no-alloc call 3 of 3: a 6000-token cut cluster (scores through the scratch's cut area)")
    sizes, G, budget, n_sink, recent = [1000, 6000, 5000], 4, 3000, 16, 9
    k0, v0, cen, labels = synth.make_planted_groups(61, sizes, n_sink=n_sink, extra_rows=recent)
    nc3 = n_sink + sum(sizes)
    init = np.array([int(np.nonzero(labels == g)[0][0]) for g in range(3)], np.int32)
    st = pipeline.prefill_unit(k0, nc3, init, 3, 2, n_sink=n_sink, v_bits=v0)
    dirs = cen / np.linalg.norm(cen, axis=1, keepdims=True)
    qv = 2.0 * dirs[0] + 1.0 * dirs[1] + 0.05 * np.random.default_rng(62).standard_normal((G, D))
    q3 = synth.f64_to_bf16_bits(qv)[None]
    L3 = gpu_layer(k0[None], v0[None], G, 3, max_budget=budget)
    load_state(L3, [st])
    L3.set_counters(nc3 + recent, nc3)
    sel = pipeline.select_unit(q3[0], st["cmean"], st["csize"], st["offsets"], st["k_clu_bits"], budget)
    assert sel["cut"] == 1 and sel["need"] == 2000
    _compare(L3, q3, budget, G, {0: st}, k0[None], v0[None], nc3, nc3 + recent, n_sink, "call 3")


def test_noalloc_rejects_a_layer_beyond_the_limit():
    # 64 units x 131072 rows of cut-score area alone exceed 16 MiB: refused before any launch
    from semantic_cluster_sparse_amd.ckv import CkvError, CkvLayerStruct
    L = CkvLayerStruct(batch=64, n_kv_heads=1, group=4, head_dim=128, n_sink=16, n_clusters=400,
                       capacity=131072, n_total=131072, n_clustered=131072, n_pending=0)
    for name, _ in CkvLayerStruct._fields_[10:]:
        setattr(L, name, 0x100000)
    with pytest.raises(CkvError) as e:
        ckv.ckv_select_decode_noalloc(L, 0x100000, 2048, 0x100000, 0x100000, 0x100000)
    assert e.value.code == ckv.CKV_ENOSPACE and "limit" in e.value.message
