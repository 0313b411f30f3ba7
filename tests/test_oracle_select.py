"""Pins for the oracle's cluster selection (oracle/select.py).

* a hand-worked golden example of the §3.3 procedure (tests/golden/select_tiny.json);
* an independent formulation: the selection is the first ``min(budget, m)``
  tokens of the total order (cluster by descending score then index; token by
  descending q.k then position) -- written here with one ``np.lexsort``;
* the recalled count is exactly ``min(budget, m)``; selections grow with the
  budget (prefix property); budget >= m recalls everything.
"""

import json
import os

import numpy as np
import pytest

from oracle import select


def test_golden_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "select_tiny.json")))
    for case in g["cases"]:
        out = select.select_unit(np.array(g["q_heads"], float), np.array(g["mu"], float),
                                 np.array(g["sizes"]), np.array(g["offsets"]),
                                 np.array(g["k_clu"], float), case["budget"])
        assert out["positions"].tolist() == case["positions"], case
        assert out["cut"] == case["cut"] and out["need"] == case["need"], case


def _random_case(rng, k=12, d=8, empty=2):
    sizes = rng.integers(1, 9, k)
    sizes[rng.choice(k, empty, replace=False)] = 0
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    m = int(offsets[-1])
    # small integer data so exact ties occur
    k_clu = rng.integers(-2, 3, (m, d)).astype(float)
    mu = rng.integers(-2, 3, (k, d)).astype(float)
    q = rng.integers(-1, 2, (3, d)).astype(float)
    return q, mu, sizes, offsets, k_clu


def _by_total_order(q, mu, sizes, offsets, k_clu, budget):
    q_bar = q.sum(axis=0)
    k = len(sizes)
    m = int(offsets[-1])
    s = np.where(sizes > 0, mu @ q_bar, -np.inf)
    crank = np.empty(k, int)
    crank[np.lexsort((np.arange(k), -s))] = np.arange(k)
    pos = np.arange(m)
    owner = np.repeat(np.arange(k), sizes)
    ts = k_clu @ q_bar
    order = np.lexsort((pos, -ts, crank[owner]))
    return np.sort(order[:min(budget, m)])


@pytest.mark.parametrize("seed", range(25))
def test_equals_total_order_prefix(seed):
    rng = np.random.default_rng(seed)
    q, mu, sizes, offsets, k_clu = _random_case(rng)
    m = int(offsets[-1])
    prev = set()
    for budget in range(0, m + 3):
        out = select.select_unit(q, mu, sizes, offsets, k_clu, budget)
        pos = out["positions"]
        assert len(pos) == min(budget, m)
        assert np.array_equal(pos, _by_total_order(q, mu, sizes, offsets, k_clu, budget))
        assert prev <= set(pos.tolist())
        prev = set(pos.tolist())
    assert prev == set(range(m))


def test_ties_and_empty_clusters():
    # two clusters with equal score: the smaller index is visited first
    mu = np.array([[1.0, 0], [1.0, 0], [0, 1.0]])
    sizes = np.array([2, 2, 0])
    offsets = np.array([0, 2, 4, 4])
    k_clu = np.array([[1.0, 0], [1.0, 0], [1.0, 0], [1.0, 0]])
    out = select.select_unit(np.array([[1.0, 5.0]]), mu, sizes, offsets, k_clu, 3)
    assert out["order"].tolist()[:2] == [0, 1]
    assert out["positions"].tolist() == [0, 1, 2]     # tie inside cluster 1 -> smaller position
    assert out["scores"][2] == -np.inf                # empty cluster never scores


def test_negative_budget_rejected():
    q, mu, sizes, offsets, k_clu = _random_case(np.random.default_rng(0))
    with pytest.raises(ValueError):
        select.select_unit(q, mu, sizes, offsets, k_clu, -1)
