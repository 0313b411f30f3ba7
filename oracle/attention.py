"""Attention over the recalled tokens of one unit (ClusterKV article §3.1), float64.

Test infrastructure only (see ``oracle/__init__``).

§3.1 states the attention the recall feeds: ``softmax(q K^T / sqrt(d)) V``.
The attended set of a decode step is the 16 sink tokens, the recalled
clustered tokens (rows of the cluster-ordered copy, §4.1) and the recent
tokens that have not been clustered yet (§3.2 clusters new tokens only every
320 steps, so until then they belong to no cluster and are always attended).
An empty attended set yields a zero output.
"""

from __future__ import annotations

import math

import numpy as np


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """``softmax(q K^T / sqrt(d)) V`` for every query row; q [G, d], K/V [R, d]."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    if K.shape[0] == 0:
        return np.zeros((q.shape[0], V.shape[1]))
    s = (q @ K.T) / math.sqrt(q.shape[1])
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V


def attended_rows(k_tok, v_tok, k_clu, v_clu, positions, n_sink: int,
                  n_clustered: int, n_total: int):
    """Keys and values of the attended set: sinks, recalled rows, recent rows."""
    pos = np.asarray(positions, np.int64)
    K = np.concatenate([k_tok[:n_sink], k_clu[pos], k_tok[n_clustered:n_total]])
    V = np.concatenate([v_tok[:n_sink], v_clu[pos], v_tok[n_clustered:n_total]])
    return K, V


def sparse_decode(q_heads, k_tok, v_tok, k_clu, v_clu, positions, n_sink: int,
                  n_clustered: int, n_total: int) -> np.ndarray:
    """Output [G, d] of every query head of the group over the attended set."""
    K, V = attended_rows(k_tok, v_tok, k_clu, v_clu, positions, n_sink,
                         n_clustered, n_total)
    return attend(q_heads, K, V)
