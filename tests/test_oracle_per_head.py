"""Pins for the oracle's per-query-head recall and decode (oracle/pipeline.py).

* each head's recall equals the independent total-order formulation of the
  single-query recall, evaluated with that head's query alone;
* when every head of a KV head carries the same query, each head's recall is
  the shared recall (the summed query is a positive multiple of it), and
  per-head decode equals the shared decode;
* heads with different queries recall different sets in general (the reading
  is not vacuous).
"""

import numpy as np
import pytest

from oracle import bf16, pipeline
from test_oracle_select import _by_total_order, _random_case


@pytest.mark.parametrize("seed", range(10))
def test_each_head_is_the_single_query_recall(seed):
    rng = np.random.default_rng(100 + seed)
    q, mu, sizes, offsets, k_clu = _random_case(rng)
    q_bits = bf16.round_rne(q)
    k_bits = bf16.round_rne(k_clu)
    for budget in (0, 5, 17, int(offsets[-1]) + 3):
        res = pipeline.select_per_head(q_bits, mu, sizes, offsets, k_bits, budget)
        assert len(res) == q.shape[0]
        for g, r in enumerate(res):
            want = _by_total_order(q[g:g + 1], mu, sizes, offsets, k_clu, budget)
            assert r["positions"].tolist() == want.tolist(), (g, budget)


def test_identical_heads_reduce_to_the_shared_recall():
    rng = np.random.default_rng(7)
    _, mu, sizes, offsets, k_clu = _random_case(rng, k=16, d=8, empty=3)
    q0 = rng.integers(-2, 3, 8).astype(float)
    q = np.tile(q0, (4, 1))
    q_bits, k_bits = bf16.round_rne(q), bf16.round_rne(k_clu)
    m = int(offsets[-1])
    v_bits = bf16.round_rne(rng.standard_normal((m + 16, 8)))
    k_tok = bf16.round_rne(rng.integers(-2, 3, (m + 16, 8)).astype(float))
    for budget in (3, 11, 30):
        shared = pipeline.select_unit(q_bits, mu, sizes, offsets, k_bits, budget)
        per = pipeline.select_per_head(q_bits, mu, sizes, offsets, k_bits, budget)
        for r in per:
            assert r["positions"].tolist() == shared["positions"].tolist()
        o_shared = pipeline.decode_unit(q_bits, k_tok, v_bits, k_bits, v_bits[16:16 + m], shared["positions"],
                                        16, 16 + m, 16 + m)
        o_per = pipeline.decode_per_head(q_bits, k_tok, v_bits, k_bits, v_bits[16:16 + m],
                                         [r["positions"] for r in per], 16, 16 + m, 16 + m)
        assert np.allclose(o_per, o_shared, rtol=0, atol=1e-12)


def test_different_heads_recall_different_sets():
    rng = np.random.default_rng(11)
    _, mu, sizes, offsets, k_clu = _random_case(rng, k=16, d=8, empty=0)
    q = np.eye(8)[:4] * 2.0
    res = pipeline.select_per_head(bf16.round_rne(q), mu, sizes, offsets, bf16.round_rne(k_clu), 10)
    assert len({tuple(r["positions"].tolist()) for r in res}) > 1
