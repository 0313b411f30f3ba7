"""Cluster-granularity recall for one unit (ClusterKV article §3.3), float64.

Test infrastructure only (see ``oracle/__init__``).

The article's selection procedure: score every cluster by the dot product of
the query with its centroid, visit clusters from the highest score down, take
whole clusters while they fit in what is left of the budget, and from the
first cluster that does not fit take only its best tokens by query-key dot
product to fill the budget exactly, then stop.  §3.1 motivates ranking by
``q . mu``: for a tight cluster ``sum_i exp(q . k_i) ~ n exp(q . mu)``.

Readings taken where the page is silent, ambiguous or garbled:

* GQA: one selection per KV head, scored with the sum of the group's query
  heads ``q_bar = sum_h q_h`` (the budget is a per-head KV budget; with one
  query head per KV head this is the page's single query).
* The partial fill takes the *highest* ``q_bar . k`` (the printed listing's
  ascending sort followed by a prefix slice would keep the least relevant
  tokens, contradicting §3.1 and "top-k").
* Ties: clusters with equal score in ascending cluster index; tokens with
  equal score in ascending position (= ascending token id, since positions
  within a cluster follow token order).
* The budget counts recalled clustered tokens only; the 16 sinks and the
  not-yet-clustered recent tokens are attended on top.  The recalled count is
  exactly ``min(budget, m)``.
* An empty cluster has no mean; it scores ``-inf`` and contributes nothing.
* Ranking uses unscaled dot products (a positive scale cannot change an
  order).
"""

from __future__ import annotations

import numpy as np


def group_query(q_heads: np.ndarray) -> np.ndarray:
    """``q_bar = sum_h q_h`` over the GQA group, float64."""
    return np.asarray(q_heads, np.float64).sum(axis=0)


def cluster_scores(q_bar: np.ndarray, mu: np.ndarray, sizes: np.ndarray) -> np.ndarray:
    """``s_j = q_bar . mu_j``, ``-inf`` for empty clusters."""
    s = np.asarray(mu, np.float64) @ q_bar
    return np.where(np.asarray(sizes) > 0, s, -np.inf)


def select_unit(q_heads, mu, sizes, offsets, k_clu, budget: int) -> dict:
    """Select ``min(budget, m)`` cluster-order positions for one unit.

    ``q_heads`` [G, d], ``mu`` [K, d], ``sizes`` [K], ``offsets`` [K+1],
    ``k_clu`` [m, d] (keys in cluster order), all float64 values.
    Returns ``positions`` (ascending), the visit ``order`` of the clusters,
    the ``cut`` cluster (-1 when every cluster fits), ``need`` (tokens taken
    from the cut cluster), and the ``scores``.
    """
    if budget < 0:
        raise ValueError("budget must be >= 0")
    sizes = np.asarray(sizes, np.int64)
    offsets = np.asarray(offsets, np.int64)
    k = sizes.shape[0]
    m = int(offsets[-1])
    q_bar = group_query(q_heads)
    s = cluster_scores(q_bar, mu, sizes)
    # visit order: score descending, then cluster index ascending
    order = np.lexsort((np.arange(k), -s))
    remaining = min(int(budget), m)
    picked = []
    cut, need = -1, 0
    for j in order:
        lo, hi = int(offsets[j]), int(offsets[j + 1])
        if hi - lo <= remaining:
            picked.append(np.arange(lo, hi))
            remaining -= hi - lo
            continue
        pos = np.arange(lo, hi)
        ts = np.asarray(k_clu, np.float64)[pos] @ q_bar
        best = np.lexsort((pos, -ts))[:remaining]
        picked.append(pos[best])
        cut, need = int(j), remaining
        break
    positions = np.sort(np.concatenate(picked)) if picked else np.zeros(0, np.int64)
    return dict(positions=positions.astype(np.int64), order=order, cut=cut,
                need=need, scores=s, q_bar=q_bar)
