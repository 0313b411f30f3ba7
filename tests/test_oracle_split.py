"""Pins for the oracle's drift test, drift split and reserved slots
(oracle/kmeans.py ``drift``, ``split``, ``init_directions``; ClusterKV article
§3.2, decoding-phase updates).

What fixes the oracle here, independently of its own code:
* drift equals the brute-force mean cosine distance of the members to the
  exact centre direction (``math.fsum`` over the members); identical members
  give 0, a pair of antipodal members gives 1;
* two planted, well separated groups merged into one cluster are separated
  exactly by one split, the smaller group moving to the empty slot;
* a threshold above every drift, or no empty slot, changes no label;
* with fewer empty slots than candidates the most drifted cluster is served
  first, and equal drifts go to the smaller index;
* the seed is the brute-force least-similar member; equal seeds go to the
  earliest token;
* labels move only from a split cluster to its slot; sizes, sums and
  directions equal a from-scratch recomputation from the labels;
* Lloyd with reserved slots (init index -1) equals Lloyd without them when no
  key scores negative against every live direction, and a key that does
  lands in the first reserved slot.
"""

import math

import numpy as np
import pytest

from oracle import bf16, kmeans
from synth import f64_to_bf16_bits


def _bf16(v):
    return bf16.widen(f64_to_bf16_bits(np.asarray(v, np.float64)))


def _state(x, a, k):
    """A consistent clustering state for labels ``a``: sums from scratch, bf16 directions."""
    a = np.asarray(a, np.int64)
    S, M, n = kmeans.unit_sums(x, a, k)
    c = kmeans.directions(S, n, np.zeros((k, x.shape[1])))
    return dict(assign=a, cdir=c, csum=S, msum=M, csize=n)


def _brute_drift(x, a, j):
    members = [i for i in range(len(a)) if a[i] == j]
    units = []
    for i in members:
        nr = math.sqrt(math.fsum(v * v for v in x[i]))
        units.append([v / nr for v in x[i]] if nr > 0 else [0.0] * x.shape[1])
    S = [math.fsum(u[t] for u in units) for t in range(x.shape[1])]
    ns = math.sqrt(math.fsum(v * v for v in S))
    if ns == 0:
        return 1.0
    return math.fsum(1.0 - math.fsum(u[t] * S[t] / ns for t in range(len(S))) for u in units) / len(units)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_drift_matches_bruteforce_mean_distance(seed):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((60, 16)) + 2.0 * rng.standard_normal(16))
    a = rng.integers(0, 5, size=60)
    S, _, n = kmeans.unit_sums(x, a, 6)
    dr = kmeans.drift(S, n)
    for j in range(5):
        if n[j]:
            assert abs(dr[j] - _brute_drift(x, a, j)) < 1e-12
            assert 0.0 <= dr[j] <= 1.0
    assert np.isnan(dr[5])


def test_drift_identical_and_antipodal_members():
    v = _bf16(np.arange(1, 9, dtype=np.float64))
    x = np.stack([v, v, v, -v])
    S, _, n = kmeans.unit_sums(x, np.array([0, 0, 0, 1]), 2)
    dr = kmeans.drift(S, n)
    assert abs(dr[0]) < 1e-15            # identical members: no spread
    assert abs(dr[1]) < 1e-15            # a singleton
    S2, _, n2 = kmeans.unit_sums(x[2:], np.array([0, 0]), 1)
    assert kmeans.drift(S2, n2)[0] == 1.0  # x and -x cancel: |S| = 0


def _two_groups(rng, na, nb, d=16):
    ea = np.zeros(d)
    ea[0] = 1.0
    eb = np.zeros(d)
    eb[1] = 1.0
    xa = 4.0 * ea + 0.1 * rng.standard_normal((na, d))
    xb = 4.0 * eb + 0.1 * rng.standard_normal((nb, d))
    return _bf16(np.concatenate([xa, xb]))


@pytest.mark.parametrize("seed", [0, 1])
def test_split_separates_two_planted_groups(seed):
    rng = np.random.default_rng(seed)
    na, nb = 30, 12
    x = _two_groups(rng, na, nb)
    order = rng.permutation(na + nb)          # interleave the groups in token order
    x = x[order]
    group_b = order >= na
    st = _state(x, np.zeros(na + nb), 2)      # one cluster holds both, slot 1 empty
    assert kmeans.drift(st["csum"], st["csize"])[0] > 0.2
    out = kmeans.split(st, x, threshold=0.1)
    assert out["pairs"] == [(0, 1)]
    # the smaller group (b) is farther from the pooled direction: it moves out
    assert np.array_equal(out["assign"], group_b.astype(np.int64))
    assert group_b[out["seeds"][0]]
    dr = kmeans.drift(out["csum"], out["csize"])
    assert dr[0] < 0.01 and dr[1] < 0.01


def test_split_noop_above_threshold_and_without_free_slot():
    rng = np.random.default_rng(3)
    x = _two_groups(rng, 20, 10)
    st = _state(x, np.zeros(30), 2)
    dmax = kmeans.drift(st["csum"], st["csize"])[0]
    out = kmeans.split(st, x, threshold=dmax)  # strictly above is needed
    assert out["pairs"] == [] and np.array_equal(out["assign"], st["assign"])
    full = _state(x, np.r_[np.zeros(29), 1], 2)  # both slots occupied
    out = kmeans.split(full, x, threshold=0.0)
    assert out["pairs"] == [] and np.array_equal(out["assign"], full["assign"])
    assert np.array_equal(out["csize"], full["csize"])


def test_split_most_drifted_first_and_drift_ties():
    rng = np.random.default_rng(4)
    d = 16
    tight = _bf16(np.r_[5.0, np.zeros(d - 1)] + 0.05 * rng.standard_normal((10, d)))
    loose = _two_groups(rng, 10, 10)
    x = np.concatenate([tight, loose])
    a = np.r_[np.zeros(10), np.ones(20)]
    st = _state(x, a, 3)
    dr = kmeans.drift(st["csum"], st["csize"])
    assert dr[1] > dr[0] > 0
    out = kmeans.split(st, x, threshold=0.0)   # both are candidates, one free slot
    assert out["pairs"] == [(1, 2)]
    assert np.all(out["assign"][:10] == 0)
    # equal drifts: cluster 1 holds the negated keys of cluster 0, so |S| and n agree exactly
    x2 = np.concatenate([loose, -loose])
    st2 = _state(x2, np.r_[np.zeros(20), np.ones(20)], 3)
    dr2 = kmeans.drift(st2["csum"], st2["csize"])
    assert dr2[0] == dr2[1]
    out2 = kmeans.split(st2, x2, threshold=0.0)
    assert out2["pairs"] == [(0, 2)]
    assert np.all(out2["assign"][20:] == 1)


def test_split_seed_is_least_similar_member_and_ties_take_earliest():
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((25, 16)) + np.r_[3.0, np.zeros(15)])
    st = _state(x, np.zeros(25), 2)
    out = kmeans.split(st, x, threshold=-1.0)
    c = st["cdir"][0]
    cos = [math.fsum(x[i] * c) / math.sqrt(math.fsum(x[i] * x[i])) for i in range(25)]
    assert out["seeds"] == [int(np.argmin(cos))]
    # duplicate the seed row earlier in token order: the earlier copy is the seed
    s = out["seeds"][0]
    x_dup = x.copy()
    x_dup[0] = x[s]
    st_dup = _state(x_dup, np.zeros(25), 2)
    cd = st_dup["cdir"][0]
    cos_d = np.array([math.fsum(x_dup[i] * cd) / math.sqrt(math.fsum(x_dup[i] * x_dup[i])) for i in range(25)])
    lo = np.flatnonzero(cos_d == cos_d.min())
    assert len(lo) >= 2 and lo[0] == 0
    assert kmeans.split(st_dup, x_dup, threshold=-1.0)["seeds"] == [0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_split_invariants_on_random_state(seed):
    rng = np.random.default_rng(seed)
    m, k, live = 200, 12, 8
    x = _bf16(rng.standard_normal((m, 16)) + rng.standard_normal(16))
    st = _state(x, rng.integers(0, live, size=m), k)
    dr = kmeans.drift(st["csum"], st["csize"])
    tau = float(np.nanmedian(dr[:live]))
    out = kmeans.split(st, x, threshold=tau)
    cands = sorted([j for j in range(live) if st["csize"][j] >= 2 and dr[j] > tau], key=lambda j: (-dr[j], j))
    assert [p[0] for p in out["pairs"]] == cands[:k - live]
    assert [p[1] for p in out["pairs"]] == list(range(live, live + len(out["pairs"])))
    moved = out["assign"] != st["assign"]
    pair_of = dict(out["pairs"])
    for i in np.flatnonzero(moved):
        assert pair_of[int(st["assign"][i])] == out["assign"][i]
    for (j, f), s in zip(out["pairs"], out["seeds"]):
        assert st["assign"][s] == j and out["assign"][s] == f
    assert out["csize"].sum() == m
    assert np.array_equal(out["csize"], np.bincount(out["assign"], minlength=k))
    S, M, n = kmeans.unit_sums(x, out["assign"], k)
    assert np.allclose(out["csum"], S, rtol=0, atol=1e-12)
    assert np.allclose(out["msum"], M, rtol=0, atol=1e-12)
    for j in range(k):
        if n[j]:
            u = S[j] / np.linalg.norm(S[j])
            assert np.array_equal(out["cdir"][j], bf16.round_value(u))
        else:
            assert np.array_equal(out["cdir"][j], st["cdir"][j])
    # the members of a split cluster took the argmax over the two directions
    for (j, f) in out["pairs"]:
        cf = bf16.round_value(kmeans.normalise(x[out["seeds"][out["pairs"].index((j, f))]][None])[0])
        for i in np.flatnonzero(st["assign"] == j):
            sj = math.fsum(x[i] * st["cdir"][j])
            sf = math.fsum(x[i] * cf)
            to_f = sf > sj or (sf == sj and f < j)
            assert out["assign"][i] == (f if to_f else j)


def test_reserved_slots_do_not_change_lloyd():
    rng = np.random.default_rng(6)
    centres = 3.0 * np.abs(rng.standard_normal((6, 16))) + 1.0
    x = _bf16(centres[rng.integers(0, 6, size=300)] + 0.5 * rng.standard_normal((300, 16)))
    # every pair of keys has a positive product, so every direction (a rounded sum of
    # unit keys) scores positive against every key in every round: no outliers
    assert (x @ x.T).min() > 0
    init = rng.choice(300, size=6, replace=False)
    plain = kmeans.lloyd(x, init, 6)
    res = kmeans.lloyd(x, np.r_[init, [-1, -1, -1]], 6)
    assert np.array_equal(res["assign"], plain["assign"])
    assert np.array_equal(res["cdir"][:6], plain["cdir"])
    assert np.all(res["cdir"][6:] == 0) and np.all(res["csize"][6:] == 0)


def test_outlier_takes_the_first_reserved_slot():
    d = 8
    e = np.eye(d)
    x = _bf16(np.stack([e[0], e[0] + 0.1 * e[2], e[1], e[1] + 0.1 * e[3], -e[0] - e[1]]))
    out = kmeans.lloyd(x, np.array([0, 2, -1, -1]), 1)
    assert list(out["assign"]) == [0, 0, 1, 1, 2]
    c = kmeans.init_directions(x, np.array([0, 2, -1, -1]))
    assert np.all(c[2:] == 0)
    assert np.array_equal(c[0], bf16.round_value(kmeans.normalise(x[:1])[0]))
