"""GPU parity of the library-drawn initial centroid indices (ckv_init_indices)
and of the seeded prefill (ckv_cluster_prefill with a seed) against the oracle.

The indices must equal the oracle's Floyd / SplitMix64 draw bit for bit; the
seeded prefill, then recall and decode, must meet the usual bars against the
oracle started from those same (oracle-drawn) indices.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import (MISMATCH_FRACTION, check_decode, check_state, compare_selection, dev_bf16, gpu_layer,
                      say)
from oracle import bf16, init, pipeline

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

from semantic_cluster_sparse_amd.layer import Layer  # noqa: E402

D = 128


@pytest.mark.parametrize("units,n_sink,m,K,seed", [
    (1, 16, 2032, 24, 0),
    (64, 16, 32752, 400, 2 ** 64 - 3),   # seed + unit wraps around 2^64
    (3, 0, 5000, 1024, 77),              # the largest K
    (5, 16, 40, 40, 9),                  # K = m: every index, in Floyd's order
    (4, 16, 1100, 1024, 3),              # K near m: most draws' targets already taken, long chains
    (2, 0, 130, 128, 11),
    (2, 5, 1, 1, 123456789),
    (1, 16, 600000, 50, 5),              # beyond the LDS bitmap: the draws' list is scanned instead
])
def test_init_indices_match_oracle(units, n_sink, m, K, seed):
    say(f"case: init draw, {units} units, m {m}, K {K}, seed {seed}")
    n = n_sink + m
    L = Layer(batch=units, n_kv_heads=1, group=1, n_clusters=K, capacity=n + 1, n_sink=n_sink, incremental=False)
    got = L.init_indices(n, seed).cpu().numpy()
    for u in range(units):
        want = init.init_indices(seed, u, m, K)
        assert got[u].tolist() == want, f"unit {u}"


def test_seeded_prefill_single_head_end_to_end():
    cfg = synth.CONFIGS["single-head-2k"]
    seed, G = 2024, 4
    say(f"case: seeded prefill {cfg.name}, seed {seed}, then recall and decode")
    k, v, cen = synth.make_layer_inputs(cfg)
    q = synth.make_queries(cfg.query_seed, cen, G)
    L = gpu_layer(k, v, G, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, seed)
    qd = dev_bf16(q)
    sp = torch.zeros((1, cfg.budget), dtype=torch.int32, device="cuda")
    cn = torch.zeros((1,), dtype=torch.int32, device="cuda")
    out = torch.zeros((1, G, D), dtype=torch.float32, device="cuda")
    L.select_decode(qd, cfg.budget, sp, cn, out)
    torch.cuda.synchronize()
    idx = np.array(init.init_indices(seed, 0, cfg.m, cfg.n_clusters))
    ora = pipeline.prefill_unit(k[0], cfg.n_tokens, idx, cfg.n_clusters, cfg.iters, v_bits=v[0], history=True)
    x = bf16.widen(k[0][16:cfg.n_tokens])
    assert check_state(L, 0, ora, x, ora["history"][-2][1], tag="seeded") == 0
    sel = pipeline.select_unit(q[0], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], cfg.budget)
    spn, cnn = sp.cpu().numpy(), cn.cpu().numpy()
    diff = compare_selection(L, 0, spn, cnn, ora, sel, cfg.budget)
    assert check_decode(out.cpu().numpy()[0], q[0], k[0], v[0], ora, spn[0], cnn[0], sel, diff, 16, cfg.n_tokens,
                        cfg.n_tokens, tag="unit 0:") == 1


def test_seeded_prefill_llama_layer():
    cfg = synth.CONFIGS["llama8b-layer-32k"]
    seed = 31337
    say(f"case: seeded prefill {cfg.name} ({cfg.units} units), seed {seed}; sampled units 0, 5")
    k, v, cen = synth.make_layer_inputs(cfg)
    q = synth.make_queries(cfg.query_seed, cen, cfg.group)
    L = gpu_layer(k, v, cfg.group, cfg.n_clusters, max_budget=cfg.budget)
    L.prefill(cfg.n_tokens, cfg.iters, seed)
    qd = dev_bf16(q)
    sp = torch.zeros((cfg.units, cfg.budget), dtype=torch.int32, device="cuda")
    cn = torch.zeros((cfg.units,), dtype=torch.int32, device="cuda")
    out = torch.zeros((cfg.units, cfg.group, D), dtype=torch.float32, device="cuda")
    L.select_decode(qd, cfg.budget, sp, cn, out)
    torch.cuda.synchronize()
    spn, cnn, og = sp.cpu().numpy(), cn.cpu().numpy(), out.cpu().numpy()
    compared = 0
    for u in (0, 5):
        idx = np.array(init.init_indices(seed, u, cfg.m, cfg.n_clusters))
        ora = pipeline.prefill_unit(k[u], cfg.n_tokens, idx, cfg.n_clusters, cfg.iters, v_bits=v[u], history=True)
        x = bf16.widen(k[u][16:cfg.n_tokens])
        mism = check_state(L, u, ora, x, ora["history"][-2][1], tag="seeded")
        assert mism <= MISMATCH_FRACTION * cfg.m
        if mism:
            continue
        sel = pipeline.select_unit(q[u], ora["cmean"], ora["csize"], ora["offsets"], ora["k_clu_bits"], cfg.budget)
        diff = compare_selection(L, u, spn, cnn, ora, sel, cfg.budget)
        compared += check_decode(og[u], q[u], k[u], v[u], ora, spn[u], cnn[u], sel, diff, 16, cfg.n_tokens,
                                 cfg.n_tokens, tag=f"unit {u}:")
    assert compared >= 1
