"""Pins for the oracle's cosine K-means (oracle/kmeans.py, oracle/pipeline.py).

What fixes the oracle here, independently of its own code:
* a hand-worked golden example (tests/golden/kmeans_tiny.json);
* assignment = brute-force argmax with exact ``math.fsum`` dot products;
  invariance under scaling a key by a power of two; K = 1; planted ties;
* exact-arithmetic Lloyd never increases the objective at either step; with
  bfloat16 directions the increase is bounded by the rounding terms;
* brute-force optimum over every labelling of tiny inputs bounds Lloyd from
  below and is reached for well-separated groups;
* the index is a stable, bijective grouping with offsets = exclusive scan;
* the scoring centroid obeys the centroid approximation of §3.1 (Jensen's
  inequality, the tight limit, and the Gaussian closed form);
* the incremental pass equals brute-force assignment plus a from-scratch
  recomputation of the running sums.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import bf16, kmeans, pipeline
from synth import f64_to_bf16_bits


def _bf16_data(rng, m, d, scale=1.0):
    return bf16.widen(f64_to_bf16_bits(rng.standard_normal((m, d)) * scale))


def _plain_unit(x):
    out = []
    for row in x:
        n = math.sqrt(math.fsum(v * v for v in row))
        out.append([v / n for v in row] if n > 0 else [0.0] * len(row))
    return np.array(out)


# ---------------------------------------------------------------- golden


def test_golden_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kmeans_tiny.json")))
    keys = np.array(g["keys"], np.float64)
    n_sink = g["n_sink"]
    k_tok = np.zeros((n_sink + len(keys), 2), np.uint16)
    k_tok[n_sink:] = bf16.round_rne(keys)
    for case in g["cases"]:
        out = pipeline.prefill_unit(k_tok, len(k_tok), np.array(g["init_idx"]), 3,
                                    case["iters"], n_sink=n_sink)
        assert out["assign"].tolist() == case["assign"]
        assert np.array_equal(out["cdir"], np.array(case["cdir"]))
        assert out["csize"].tolist() == case["csize"]
        assert np.allclose(out["cmean"], np.array(case["cmean"]), rtol=0, atol=1e-12)
        assert out["perm"].tolist() == case["perm"]
        assert out["offsets"].tolist() == case["offsets"]


# ---------------------------------------------------------------- assign


@pytest.mark.parametrize("seed", range(4))
def test_assign_bruteforce_fsum(seed):
    rng = np.random.default_rng(seed)
    m, k, d = 40, 7, 16
    x = _bf16_data(rng, m, d, 3.0)
    c = bf16.round_value(_plain_unit(rng.standard_normal((k, d))))
    a = kmeans.assign(x, c)
    for i in range(m):
        s = [math.fsum(x[i, t] * c[j, t] for t in range(d)) for j in range(k)]
        best = max(s)
        assert a[i] == s.index(best)


def test_assign_k1_scaling_and_ties():
    rng = np.random.default_rng(5)
    x = _bf16_data(rng, 64, 32)
    c1 = bf16.round_value(_plain_unit(rng.standard_normal((1, 32))))
    assert np.all(kmeans.assign(x, c1) == 0)
    c = bf16.round_value(_plain_unit(rng.standard_normal((6, 32))))
    a = kmeans.assign(x, c)
    for p in (-3, 2, 5):  # power-of-two scaling is exact in bfloat16
        assert np.array_equal(kmeans.assign(x * 2.0 ** p, c), a)
    # duplicated directions: the smaller index always wins the tie
    cd = np.concatenate([c[:3], c[:3]])
    assert np.all(kmeans.assign(x, cd) < 3)
    cd2 = np.concatenate([c[3:], c[:3], c[:3]])
    assert not np.any((kmeans.assign(x, cd2) >= 6))
    # a zero key scores 0 everywhere and goes to cluster 0
    x0 = np.zeros((1, 32))
    assert kmeans.assign(x0, c)[0] == 0
    # a key equal to a direction, with a clear margin, is assigned to it
    for j in range(6):
        assert kmeans.assign(c[j:j + 1] * 4.0, c)[0] == j


# ---------------------------------------------------------------- Lloyd


def _J(xh, a, c):
    return float(sum(1.0 - np.dot(xh[i], c[a[i]]) for i in range(len(a))))


@pytest.mark.parametrize("seed", range(3))
def test_lloyd_exact_mode_monotone(seed):
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((5, 8)) * 3
    x = centres[rng.integers(0, 5, 200)] + rng.standard_normal((200, 8))
    x = bf16.round_value(x)
    xh = _plain_unit(x)
    init = rng.choice(200, 6, replace=False)
    out = kmeans.lloyd(x, init, 12, round_bf16=False, history=True)
    hist = out["history"]
    prev = None
    for t in range(1, len(hist)):
        a_t, c_t = hist[t]
        c_prev = hist[t - 1][1]
        j_assign = _J(xh, a_t, c_prev)        # after assigning with c^(t-1)
        j_update = _J(xh, a_t, c_t)           # after updating to c^(t)
        assert j_update <= j_assign + 1e-9
        if prev is not None:
            assert j_assign <= prev + 1e-9    # assignment with c^(t-1) can only improve
        prev = j_update


@pytest.mark.parametrize("seed", range(3))
def test_lloyd_bf16_mode_bounded_by_rounding(seed):
    rng = np.random.default_rng(10 + seed)
    centres = rng.standard_normal((6, 16)) * 3
    x = bf16.round_value(centres[rng.integers(0, 6, 300)] + rng.standard_normal((300, 16)))
    xh = _plain_unit(x)
    init = rng.choice(300, 5, replace=False)
    out = kmeans.lloyd(x, init, 8, history=True)
    hist = out["history"]
    for t in range(1, len(hist)):
        a, c_t = hist[t]
        c_prev = hist[t - 1][1]
        k = c_t.shape[0]
        S = np.zeros_like(c_t)
        cnt = np.zeros(k, int)
        for i in range(len(a)):
            S[a[i]] += xh[i]
            cnt[a[i]] += 1
        eps = eta = 0.0
        for j in range(k):
            ns = math.sqrt(float(np.dot(S[j], S[j])))
            if cnt[j] == 0 or ns == 0:
                continue
            u = S[j] / ns
            eps += float(np.dot(S[j], c_t[j] - u))
            cp = c_prev[j]
            eta += float(np.dot(S[j], cp / math.sqrt(float(np.dot(cp, cp))) - cp))
        assert _J(xh, a, c_t) <= _J(xh, a, c_prev) + abs(eps) + abs(eta) + 1e-9


def test_lloyd_fixed_point():
    rng = np.random.default_rng(3)
    centres = rng.standard_normal((4, 8)) * 4
    x = bf16.round_value(centres[rng.integers(0, 4, 120)] + rng.standard_normal((120, 8)))
    out = kmeans.lloyd(x, rng.choice(120, 4, replace=False), 40)
    a = out["assign"]
    assert np.array_equal(kmeans.assign(x, out["cdir"]), a)
    again = kmeans.directions(*kmeans.unit_sums(x, a, 4)[0::2], out["cdir"])
    assert np.array_equal(again, out["cdir"])


def _best_labelling(xh, k):
    best = float("inf")
    for lab in itertools.product(range(k), repeat=len(xh)):
        val = 0.0
        for j in range(k):
            mem = [i for i in range(len(xh)) if lab[i] == j]
            if mem:
                s = xh[mem].sum(axis=0)
                val += len(mem) - math.sqrt(float(np.dot(s, s)))
        best = min(best, val)
    return best


@pytest.mark.parametrize("seed", range(6))
def test_lloyd_vs_bruteforce_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    m, k = 7, 3
    x = bf16.round_value(rng.standard_normal((m, 3)))
    xh = _plain_unit(x)
    jstar = _best_labelling(xh, k)
    out = kmeans.lloyd(x, rng.choice(m, k, replace=False), 10, round_bf16=False)
    S, _, n = kmeans.unit_sums(x, out["assign"], k)
    j_lloyd = float(sum(n[j] - math.sqrt(float(np.dot(S[j], S[j]))) for j in range(k)))
    assert j_lloyd >= jstar - 1e-12


def test_lloyd_reaches_optimum_on_separated_groups():
    rng = np.random.default_rng(7)
    dirs = np.eye(3)
    groups = [dirs[g] * 5 + rng.standard_normal((3, 3)) * 0.05 for g in range(3)]
    x = bf16.round_value(np.concatenate(groups))
    xh = _plain_unit(x)
    out = kmeans.lloyd(x, np.array([0, 3, 6]), 5, round_bf16=False)
    S, _, n = kmeans.unit_sums(x, out["assign"], 3)
    j_lloyd = float(sum(n[j] - math.sqrt(float(np.dot(S[j], S[j]))) for j in range(3)))
    assert out["assign"].tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2]
    assert abs(j_lloyd - _best_labelling(xh, 3)) < 1e-12


# ---------------------------------------------------------------- index


@pytest.mark.parametrize("seed", range(3))
def test_index_is_stable_bijection(seed):
    rng = np.random.default_rng(seed)
    k, m, n_sink = 9, 500, 16
    a = rng.integers(0, k, m)
    a[a == 4] = 5   # leave cluster 4 empty
    perm, off = kmeans.build_index(a, k, n_sink)
    assert sorted(perm.tolist()) == list(range(n_sink, n_sink + m))
    counts = [int(np.sum(a == j)) for j in range(k)]
    assert off.tolist() == [0] + list(np.cumsum(counts))
    for j in range(k):
        ids = perm[off[j]:off[j + 1]]
        assert all(a[i - n_sink] == j for i in ids)
        assert list(ids) == sorted(ids)
    assert off[-1] == m and off[4] == off[5]


# ---------------------------------------------------------------- scoring centroid (§3.1)


def test_centroid_jensen_and_tight_limit():
    rng = np.random.default_rng(11)
    for sigma in (1.0, 0.3, 0.1, 0.01, 0.001):
        c = rng.standard_normal(16)
        x = c + sigma * rng.standard_normal((50, 16))
        S, M, n = kmeans.unit_sums(x, np.zeros(50, int), 1)
        mu = kmeans.scoring_centroids(M, n)[0]
        q = rng.standard_normal(16) * 0.5
        lhs = np.logaddexp.reduce(x @ q)            # log sum_i exp(q.x_i)
        rhs = math.log(50) + float(mu @ q)         # log n exp(q.mu)
        assert lhs >= rhs - 1e-12                  # Jensen, exact
        if sigma <= 0.001:
            assert lhs - rhs < 1e-5                # tight cluster: ratio -> 1


def test_centroid_gaussian_closed_form():
    # members c + sigma*eps_i: E[sum exp(q.x_i) / (n exp(q.mu))] = exp(s^2 |q|^2 (1-1/n) / 2)
    rng = np.random.default_rng(12)
    n, d, sigma, trials = 20, 8, 0.25, 4000
    q = rng.standard_normal(d)
    q *= 2.0 / np.linalg.norm(q)                    # sigma*|q| = 0.5
    ratios = np.empty(trials)
    for t in range(trials):
        x = rng.standard_normal(d) + sigma * rng.standard_normal((n, d))
        _, M, cnt = kmeans.unit_sums(x, np.zeros(n, int), 1)
        mu = kmeans.scoring_centroids(M, cnt)[0]
        ratios[t] = np.exp(x @ q - mu @ q).sum() / n
    expect = math.exp(sigma ** 2 * float(q @ q) * (1 - 1 / n) / 2)
    stderr = ratios.std() / math.sqrt(trials)
    assert abs(ratios.mean() - expect) < 5 * stderr + 1e-3


# ---------------------------------------------------------------- incremental


def test_incremental_matches_bruteforce_and_recompute():
    rng = np.random.default_rng(21)
    k, d = 6, 16
    centres = rng.standard_normal((8, d)) * 3
    x_old = bf16.round_value(centres[rng.integers(0, 8, 200)] + rng.standard_normal((200, d)))
    state = kmeans.lloyd(x_old, rng.choice(200, k, replace=False), 5, round_bf16=True)
    x_new = bf16.round_value(centres[rng.integers(0, 8, 40)] + rng.standard_normal((40, d)))
    out = kmeans.incremental(state, x_new)
    # brute-force labels of the new keys against the pre-update directions
    for i in range(40):
        s = [math.fsum(x_new[i, t] * state["cdir"][j, t] for t in range(d)) for j in range(k)]
        assert out["new_assign"][i] == s.index(max(s))
    assert np.array_equal(out["assign"][:200], state["assign"])
    # running sums equal a from-scratch recomputation over all members
    x_all = np.concatenate([x_old, x_new])
    xh = _plain_unit(x_all)
    for j in range(k):
        mem = out["assign"] == j
        assert out["csize"][j] == mem.sum()
        assert np.allclose(out["csum"][j], xh[mem].sum(axis=0), rtol=0, atol=1e-12)
        assert np.allclose(out["msum"][j], x_all[mem].sum(axis=0), rtol=0, atol=1e-10)
    # touched clusters get the direction of their new unit-key sum, others keep theirs
    touched = np.bincount(out["new_assign"], minlength=k) > 0
    for j in range(k):
        if touched[j]:
            u = out["csum"][j] / np.linalg.norm(out["csum"][j])
            assert np.array_equal(out["cdir"][j], bf16.round_value(u))
        else:
            assert np.array_equal(out["cdir"][j], state["cdir"][j])


def test_incremental_empty_is_noop():
    rng = np.random.default_rng(22)
    x = bf16.round_value(rng.standard_normal((50, 8)))
    state = kmeans.lloyd(x, np.arange(4), 3)
    out = kmeans.incremental(state, np.zeros((0, 8)))
    for key in ("cdir", "csum", "msum", "csize", "assign"):
        assert np.array_equal(out[key], state[key])
