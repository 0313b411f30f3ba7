"""Per-unit end-to-end oracle: prefill clustering, incremental pass, recall, decode.

Test infrastructure only (see ``oracle/__init__``).

Inputs are bfloat16 bit patterns (uint16) exactly as the GPU receives them;
outputs are float64 values, plus bfloat16 bit patterns where the method itself
rounds (the centroid directions).  One *unit* is one KV head of one sequence
of one layer; units never interact.
"""

from __future__ import annotations

import numpy as np

from . import attention, bf16, kmeans, select


def prefill_unit(k_bits: np.ndarray, n: int, init_idx, n_clusters: int, iters: int,
                 n_sink: int = kmeans.N_SINK, v_bits: np.ndarray | None = None,
                 history: bool = False) -> dict:
    """Cluster tokens ``[n_sink, n)`` of one unit (ClusterKV article §3.2, §4.1).

    Returns the final labels ``assign`` [m], directions ``cdir`` (values) and
    ``cdir_bits``, running sums ``csum``/``msum``, sizes ``csize``, scoring
    centroids ``cmean``, the index ``perm``/``offsets`` and the
    cluster-ordered key (and value) rows ``k_clu_bits``/``v_clu_bits``.
    """
    m = n - n_sink
    if not (1 <= n_clusters <= m):
        raise ValueError("need 1 <= K <= m")
    x = bf16.widen(k_bits[n_sink:n])
    out = kmeans.lloyd(x, init_idx, iters, history=history)
    perm, offsets = kmeans.build_index(out["assign"], n_clusters, n_sink)
    out["cdir_bits"] = bf16.round_rne(out["cdir"])
    out["cmean"] = kmeans.scoring_centroids(out["msum"], out["csize"])
    out["perm"] = perm
    out["offsets"] = offsets
    out["k_clu_bits"] = np.asarray(k_bits)[perm]
    if v_bits is not None:
        out["v_clu_bits"] = np.asarray(v_bits)[perm]
    out["n_clustered"] = n
    return out


def incremental_unit(state: dict, k_bits: np.ndarray, n_total: int,
                     n_sink: int = kmeans.N_SINK, v_bits: np.ndarray | None = None) -> dict:
    """Cluster tokens ``[state['n_clustered'], n_total)`` against the existing clusters."""
    lo = state["n_clustered"]
    x_new = bf16.widen(k_bits[lo:n_total])
    out = kmeans.incremental(state, x_new)
    k = out["cdir"].shape[0]
    perm, offsets = kmeans.build_index(out["assign"], k, n_sink)
    out["cdir_bits"] = bf16.round_rne(out["cdir"])
    out["cmean"] = kmeans.scoring_centroids(out["msum"], out["csize"])
    out["perm"] = perm
    out["offsets"] = offsets
    out["k_clu_bits"] = np.asarray(k_bits)[perm]
    if v_bits is not None:
        out["v_clu_bits"] = np.asarray(v_bits)[perm]
    out["n_clustered"] = n_total
    return out


def split_unit(state: dict, k_bits: np.ndarray, threshold: float, n_sink: int = kmeans.N_SINK,
               v_bits: np.ndarray | None = None) -> dict:
    """Drift-triggered split of the clusters of tokens ``[n_sink, state['n_clustered'])``
    (ClusterKV article §3.2), then the cluster-contiguous index and rows (§4.1)."""
    n = state["n_clustered"]
    x = bf16.widen(k_bits[n_sink:n])
    out = kmeans.split(state, x, threshold)
    k = out["cdir"].shape[0]
    perm, offsets = kmeans.build_index(out["assign"], k, n_sink)
    out["cdir_bits"] = bf16.round_rne(out["cdir"])
    out["cmean"] = kmeans.scoring_centroids(out["msum"], out["csize"])
    out["perm"] = perm
    out["offsets"] = offsets
    out["k_clu_bits"] = np.asarray(k_bits)[perm]
    if v_bits is not None:
        out["v_clu_bits"] = np.asarray(v_bits)[perm]
    out["n_clustered"] = n
    return out


def select_unit(q_bits: np.ndarray, cmean: np.ndarray, csize, offsets,
                k_clu_bits: np.ndarray, budget: int) -> dict:
    """Recall for one unit: ``q_bits`` [G, d] bf16 bits, ``cmean`` float values."""
    return select.select_unit(bf16.widen(q_bits), cmean, csize, offsets,
                              bf16.widen(k_clu_bits), budget)


def decode_unit(q_bits, k_tok_bits, v_tok_bits, k_clu_bits, v_clu_bits, positions,
                n_sink: int, n_clustered: int, n_total: int) -> np.ndarray:
    """Attention output [G, d] (float64) over sinks + recalled rows + recent rows."""
    return attention.sparse_decode(
        bf16.widen(q_bits), bf16.widen(k_tok_bits), bf16.widen(v_tok_bits),
        bf16.widen(k_clu_bits), bf16.widen(v_clu_bits), positions,
        n_sink, n_clustered, n_total)


def select_per_head(q_bits: np.ndarray, cmean: np.ndarray, csize, offsets,
                    k_clu_bits: np.ndarray, budget: int) -> list[dict]:
    """Per-query-head recall, the other grouped-query reading of the ClusterKV
    article's §3.3: the recall is stated for one query, so every query head g
    runs it with q_g alone (no sum over the heads of a KV head).  One result per
    row of ``q_bits`` [G, d]."""
    return [select_unit(q_bits[g:g + 1], cmean, csize, offsets, k_clu_bits, budget)
            for g in range(q_bits.shape[0])]


def decode_per_head(q_bits, k_tok_bits, v_tok_bits, k_clu_bits, v_clu_bits, positions_per_head,
                    n_sink: int, n_clustered: int, n_total: int) -> np.ndarray:
    """Attention output [G, d]: head g attends to the sinks, its own recalled rows
    and the recent rows."""
    return np.stack([decode_unit(q_bits[g:g + 1], k_tok_bits, v_tok_bits, k_clu_bits, v_clu_bits,
                                 positions_per_head[g], n_sink, n_clustered, n_total)[0]
                     for g in range(q_bits.shape[0])])
