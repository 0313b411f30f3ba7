"""Cosine K-means of one unit's keys (prefill and incremental), float64.

Test infrastructure only (see ``oracle/__init__``).

Follows the ClusterKV article, §3.2: at prefill the first 16 tokens are kept
out of the clustering, and the remaining keys are clustered by K-means under
cosine distance; during decoding, newly generated tokens are clustered
incrementally with an online K-means variant every 320 tokens.  §3.1 gives the
centroid as the plain mean of the member keys; §4.1 stores each cluster's
tokens contiguously.

Readings taken where the pages are silent:

* Two centroid roles (§3.1 vs §3.2): the *direction* ``c~_j`` drives the
  cosine assignment and is the spherical-K-means update
  ``bf16(S_j / |S_j|)`` with ``S_j`` the sum of the members' unit keys; the
  *scoring centroid* ``mu_j = M_j / n_j`` is the raw mean of §3.1, with
  ``M_j`` the plain sum of the members' keys.
* Assignment is ``argmax_j x . c~_j``.  Because ``|x|`` is fixed per key this
  is the cosine argmax.  Ties go to the smallest ``j``.  A zero key scores 0
  everywhere and so lands in cluster 0.
* Initial directions are ``bf16(x_I / |x_I|)`` for ``K`` distinct indices
  ``I`` drawn by the caller (a random draw, passed in).
* Exactly ``T`` assign+update rounds, no early stop.
* An empty cluster, or one whose unit-key sum is zero, keeps its previous
  direction; its scoring centroid is undefined (reported as 0, size 0).
* Incremental pass: the new keys are assigned to the current directions, then
  folded into ``S``, ``M``, ``n``; the touched clusters' directions and means
  are refreshed; old tokens are never reassigned and ``K`` does not change.
"""

from __future__ import annotations

import numpy as np

from . import bf16

N_SINK = 16


def normalise(x: np.ndarray) -> np.ndarray:
    """Unit keys ``x / |x|`` (float64); a zero key stays zero."""
    x = np.asarray(x, dtype=np.float64)
    norms = np.sqrt(np.sum(x * x, axis=1))
    out = np.zeros_like(x)
    nz = norms > 0
    out[nz] = x[nz] / norms[nz, None]
    return out


def assign(x: np.ndarray, cdir: np.ndarray) -> np.ndarray:
    """Cosine assignment (ClusterKV article §3.2): ``argmax_j x . c~_j``.

    ``x`` [m, d] and ``cdir`` [K, d] hold bfloat16 values in float64, so every
    product is exact; ``np.argmax`` returns the first (smallest-index) maximum.
    """
    if x.shape[0] == 0:
        return np.zeros(0, np.int64)
    scores = np.asarray(x, np.float64) @ np.asarray(cdir, np.float64).T
    return np.argmax(scores, axis=1).astype(np.int64)


def unit_sums(x: np.ndarray, a: np.ndarray, k: int):
    """Per-cluster ``S_j = sum x^_i``, ``M_j = sum x_i`` and ``n_j`` for labels ``a``."""
    xh = normalise(x)
    d = x.shape[1]
    S = np.zeros((k, d))
    M = np.zeros((k, d))
    n = np.zeros(k, np.int64)
    for j in range(k):
        members = a == j
        n[j] = int(np.count_nonzero(members))
        if n[j]:
            S[j] = xh[members].sum(axis=0)
            M[j] = np.asarray(x, np.float64)[members].sum(axis=0)
    return S, M, n


def directions(S: np.ndarray, n: np.ndarray, prev: np.ndarray, round_bf16: bool = True):
    """Direction update ``c~_j = bf16(S_j / |S_j|)``; empty or zero-sum clusters keep ``prev``."""
    out = np.array(prev, dtype=np.float64, copy=True)
    norms = np.sqrt(np.sum(S * S, axis=1))
    ok = (n > 0) & (norms > 0)
    unit = S[ok] / norms[ok, None]
    out[ok] = bf16.round_value(unit) if round_bf16 else unit
    return out


def init_directions(x: np.ndarray, init_idx: np.ndarray, round_bf16: bool = True):
    """Initial directions from the caller's distinct indices into the clustered keys."""
    xh = normalise(x[np.asarray(init_idx, np.int64)])
    return bf16.round_value(xh) if round_bf16 else xh


def objective(x: np.ndarray, a: np.ndarray, cdir: np.ndarray) -> float:
    """Cosine K-means objective ``J = sum_i (1 - x^_i . c_{a_i})``."""
    xh = normalise(x)
    return float(np.sum(1.0 - np.sum(xh * np.asarray(cdir)[a], axis=1)))


def lloyd(x: np.ndarray, init_idx: np.ndarray, iters: int, round_bf16: bool = True,
          history: bool = False):
    """``iters`` Lloyd rounds of cosine K-means on the clustered keys ``x`` [m, d].

    Round ``t``: assign with ``c~^(t-1)``, then update to ``c~^(t)``.  Returns a
    dict with the final assignment ``assign`` (labels in ``[0, K)``), the
    final directions ``cdir`` (float64 holding bfloat16 values unless
    ``round_bf16`` is False), ``csum``/``msum``/``csize`` from the final
    assignment, and, with ``history``, every round's ``(assign, cdir)``.
    """
    if iters < 1:
        raise ValueError("at least one Lloyd round")
    k = len(init_idx)
    c = init_directions(x, init_idx, round_bf16)
    hist = [(None, c.copy())]
    a = None
    S = M = n = None
    for _ in range(iters):
        a = assign(x, c)
        S, M, n = unit_sums(x, a, k)
        c = directions(S, n, c, round_bf16)
        if history:
            hist.append((a.copy(), c.copy()))
    out = dict(assign=a, cdir=c, csum=S, msum=M, csize=n)
    if history:
        out["history"] = hist
    return out


def scoring_centroids(M: np.ndarray, n: np.ndarray) -> np.ndarray:
    """Scoring centroid ``mu_j = M_j / n_j``, the mean key of §3.1; 0 for empty clusters."""
    mu = np.zeros_like(M)
    nz = n > 0
    mu[nz] = M[nz] / n[nz, None]
    return mu


def build_index(a: np.ndarray, k: int, n_sink: int = N_SINK):
    """Cluster-contiguous index (ClusterKV article §4.1).

    ``perm[p]`` is the token id (sinks counted, so ids start at ``n_sink``)
    at cluster-order position ``p``; tokens are grouped by cluster in
    ascending cluster order and keep ascending token order inside a cluster.
    ``offsets`` [K+1] delimits cluster ``j`` as ``offsets[j]:offsets[j+1]``.
    """
    a = np.asarray(a, np.int64)
    perm = np.argsort(a, kind="stable") + n_sink
    counts = np.bincount(a, minlength=k)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return perm.astype(np.int64), offsets


def incremental(state: dict, x_new: np.ndarray, round_bf16: bool = True) -> dict:
    """Online clustering of new keys against existing clusters (ClusterKV article §3.2).

    ``state`` holds ``assign`` (labels of the already clustered keys),
    ``cdir``, ``csum``, ``msum``, ``csize``.  The new keys are assigned to
    the *current* directions, added to the running sums, and the touched
    clusters get a fresh direction (if their unit-key sum is nonzero) and
    mean.  Returns a new state with the labels of old and new keys
    concatenated in token order.
    """
    k = state["cdir"].shape[0]
    a_new = assign(x_new, state["cdir"])
    dS, dM, dn = unit_sums(x_new, a_new, k)
    S = state["csum"] + dS
    M = state["msum"] + dM
    n = state["csize"] + dn
    touched = dn > 0
    c = np.array(state["cdir"], np.float64, copy=True)
    upd = directions(S, n, c, round_bf16)
    c[touched] = upd[touched]
    return dict(assign=np.concatenate([np.asarray(state["assign"], np.int64), a_new]),
                cdir=c, csum=S, msum=M, csize=n, new_assign=a_new)
