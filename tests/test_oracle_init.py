"""Pins of the oracle's seeded initial centroid indices (oracle/init.py).

* SplitMix64 reproduces the generator's published first outputs from state 0;
* Floyd's algorithm reproduces hand-worked draws (tests/golden/init_floyd_tiny.json);
* the composed draw gives K distinct indices in [0, m), is deterministic in
  (seed, unit), differs between units, and draws every K-subset about equally
  often (Floyd's algorithm samples subsets uniformly; the insertion order is
  not uniform: the first index comes from [0, m - K]);
* K = m gives a permutation of [0, m), K = 0 an empty sample.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import init


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "init_floyd_tiny.json")) as f:
        return json.load(f)


def test_splitmix64_published_outputs(golden_dir):
    g = _golden(golden_dir)["splitmix64"]
    stream = init.splitmix64(g["state"])
    got = [next(stream) for _ in g["outputs_hex"]]
    assert got == [int(h, 16) for h in g["outputs_hex"]]


@pytest.mark.parametrize("case", ["floyd", "floyd_all"])
def test_floyd_hand_worked(golden_dir, case):
    g = _golden(golden_dir)[case]
    assert init.floyd_sample(g["m"], g["k"], iter(g["draws"])) == g["indices"]


@pytest.mark.parametrize("m,k", [(1, 1), (7, 3), (100, 100), (32752, 400), (2032, 24), (5000, 1024)])
def test_distinct_in_range_and_deterministic(m, k):
    for unit in (0, 1, 63):
        a = init.init_indices(2024, unit, m, k)
        assert len(a) == k and len(set(a)) == k
        assert all(0 <= i < m for i in a)
        assert a == init.init_indices(2024, unit, m, k)
    assert init.init_indices(2024, 0, m, k) != init.init_indices(2024, 1, m, k) or k == m


def test_k_equals_m_is_a_permutation_and_zero_is_empty():
    for m in (1, 5, 64):
        assert sorted(init.init_indices(7, 3, m, m)) == list(range(m))
    assert init.init_indices(7, 3, 10, 0) == []
    with pytest.raises(ValueError):
        init.floyd_sample(3, 4, iter([0] * 4))


def test_unit_offsets_the_state():
    # unit u of seed s draws what unit 0 of seed s + u draws
    assert init.init_indices(100, 5, 500, 40) == init.init_indices(105, 0, 500, 40)


def test_every_subset_about_equally_likely():
    m, k, n = 5, 2, 20000
    counts = {c: 0 for c in itertools.combinations(range(m), k)}
    for s in range(n):
        counts[tuple(sorted(init.init_indices(s, 0, m, k)))] += 1
    expect = n / len(counts)
    chi2 = sum((c - expect) ** 2 / expect for c in counts.values())
    # 9 degrees of freedom: P(chi2 > 27.9) = 0.001
    assert chi2 < 27.9, counts
    # the first inserted index is the first draw modulo m - K + 1: uniform over [0, m - K], never above
    first = np.bincount([init.init_indices(s, 0, m, k)[0] for s in range(n)], minlength=m)
    lo = m - k + 1
    assert np.all(first[lo:] == 0)
    assert np.all(np.abs(first[:lo] - n / lo) < 5 * np.sqrt(n / lo))
