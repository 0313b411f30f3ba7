"""Planted mistakes in the oracle must be caught by its pins.

Each case monkeypatches one plausible slip into the oracle (on the CPU) and
checks that a pin from the other test files fails on it: a dropped
normalisation, ties to the wrong index, a dropped 1/sqrt(d), a reversed
cluster order, an unstable index, recent tokens left out of the attended set,
and in the seeded init a wrong modulus, a duplicate insert and a wrong
generator constant.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, bf16, init, kmeans, pipeline, select


def _kmeans_golden_ok(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kmeans_tiny.json")))
    k_tok = np.zeros((g["n_sink"] + len(g["keys"]), 2), np.uint16)
    k_tok[g["n_sink"]:] = bf16.round_rne(np.array(g["keys"], float))
    for case in g["cases"]:
        out = pipeline.prefill_unit(k_tok, len(k_tok), np.array(g["init_idx"]), 3,
                                    case["iters"], n_sink=g["n_sink"])
        if (out["assign"].tolist() != case["assign"]
                or not np.array_equal(out["cdir"], np.array(case["cdir"]))
                or out["perm"].tolist() != case["perm"]):
            return False
    return True


def _select_golden_ok(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "select_tiny.json")))
    for case in g["cases"]:
        out = select.select_unit(np.array(g["q_heads"], float), np.array(g["mu"], float),
                                 np.array(g["sizes"]), np.array(g["offsets"]),
                                 np.array(g["k_clu"], float), case["budget"])
        if out["positions"].tolist() != case["positions"]:
            return False
    return True


def _attention_ok(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attention_tiny.json")))
    out = attention.attend(np.array(g["q_heads"]), np.array(g["keys"], float),
                           np.array(g["values"], float))
    if not np.allclose(out, np.array(g["out"], float), atol=1e-12):
        return False
    rng = np.random.default_rng(0)
    q, K, V = rng.standard_normal((2, 128)), rng.standard_normal((30, 128)), rng.standard_normal((30, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(K)[None, None].expand(1, 2, 30, 128),
        torch.from_numpy(V)[None, None].expand(1, 2, 30, 128))[0, :, 0].numpy()
    return np.allclose(attention.attend(q, K, V), ref, atol=1e-12)


def test_unplanted_oracle_passes(golden_dir):
    assert _kmeans_golden_ok(golden_dir)
    assert _select_golden_ok(golden_dir)
    assert _attention_ok(golden_dir)


def test_dropped_normalisation_is_caught(golden_dir, monkeypatch):
    monkeypatch.setattr(kmeans, "normalise", lambda x: np.asarray(x, float))
    assert not _kmeans_golden_ok(golden_dir)


def test_ties_to_largest_index_is_caught(golden_dir, monkeypatch):
    def bad_assign(x, c):
        s = np.asarray(x) @ np.asarray(c).T
        return (s.shape[1] - 1 - np.argmax(s[:, ::-1], axis=1)).astype(np.int64)
    monkeypatch.setattr(kmeans, "assign", bad_assign)
    assert not _kmeans_golden_ok(golden_dir)


def test_dropped_scale_is_caught(golden_dir, monkeypatch):
    monkeypatch.setattr(attention, "math", type("m", (), {"sqrt": staticmethod(lambda v: 1.0)}))
    assert not _attention_ok(golden_dir)


def test_reversed_cluster_order_is_caught(golden_dir, monkeypatch):
    orig = select.cluster_scores
    monkeypatch.setattr(select, "cluster_scores", lambda q, mu, s: -orig(q, mu, s))
    assert not _select_golden_ok(golden_dir)


def test_unstable_index_is_caught(golden_dir, monkeypatch):
    def bad_index(a, k, n_sink=16):
        a = np.asarray(a, np.int64)
        perm = (len(a) - 1 - np.argsort(a[::-1], kind="stable")) + n_sink
        counts = np.bincount(a, minlength=k)
        return perm, np.concatenate([[0], np.cumsum(counts)])
    monkeypatch.setattr(kmeans, "build_index", bad_index)
    assert not _kmeans_golden_ok(golden_dir)


def test_missing_recent_rows_is_caught(monkeypatch):
    k_tok = np.arange(20, dtype=float).reshape(10, 2)
    orig = attention.attended_rows
    monkeypatch.setattr(attention, "attended_rows",
                        lambda kt, vt, kc, vc, p, s, nc, nt: orig(kt, vt, kc, vc, p, s, nc, nc))
    K, _ = attention.attended_rows(k_tok, k_tok, k_tok, k_tok, [1], 2, 7, 9)
    assert len(K) != 2 + 1 + 2


def _init_golden_ok(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "init_floyd_tiny.json")))
    st = init.splitmix64(g["splitmix64"]["state"])
    if [next(st) for _ in range(3)] != [int(h, 16) for h in g["splitmix64"]["outputs_hex"]]:
        return False
    for case in ("floyd", "floyd_all"):
        c = g[case]
        if init.floyd_sample(c["m"], c["k"], iter(c["draws"])) != c["indices"]:
            return False
    return True


def test_unplanted_init_passes(golden_dir):
    assert _init_golden_ok(golden_dir)


def test_init_modulus_off_by_one_is_caught(golden_dir, monkeypatch):
    def bad(m, k, draws):
        out, seen = [], set()
        for j in range(m - k, m):
            t = next(draws) % max(j, 1)          # j instead of j + 1
            p = t if t not in seen else j
            seen.add(p)
            out.append(p)
        return out
    monkeypatch.setattr(init, "floyd_sample", bad)
    assert not _init_golden_ok(golden_dir)


def test_init_duplicate_insert_is_caught(golden_dir, monkeypatch):
    monkeypatch.setattr(init, "floyd_sample",
                        lambda m, k, draws: [next(draws) % (j + 1) for j in range(m - k, m)])
    assert not _init_golden_ok(golden_dir)


def test_init_generator_constant_is_caught(golden_dir, monkeypatch):
    monkeypatch.setattr(init, "GOLDEN_GAMMA", 0x9E3779B97F4A7C13)
    assert not _init_golden_ok(golden_dir)
