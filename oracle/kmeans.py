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
* Drift split (``split``): ``K`` is a slot count; a split moves part of a
  drifted cluster into an empty slot.  Prefill may leave slots empty on
  purpose (init index -1, zero direction).
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
    """Initial directions from the caller's distinct indices into the clustered keys.

    An index of -1 reserves the slot: its direction is the zero vector, which
    scores exactly 0 against every key, so the slot stays empty unless some
    key's best score against the live directions is negative (an outlier,
    which then gets the slot).  Reserved slots are where ``split`` puts the
    halves it creates.
    """
    idx = np.asarray(init_idx, np.int64)
    out = np.zeros((len(idx), x.shape[1]))
    live = idx >= 0
    xh = normalise(x[idx[live]])
    out[live] = bf16.round_value(xh) if round_bf16 else xh
    return out


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


def drift(S: np.ndarray, n: np.ndarray) -> np.ndarray:
    """Mean cosine distance of each cluster's members to its centre direction.

    The drift test of the ClusterKV article (§3.2, decoding-phase updates)
    compares a cluster's mean intra-cluster distance with a threshold.  Under
    cosine distance to the exact centre direction ``S_j / |S_j|`` that mean is
    ``(1/n_j) sum_i (1 - x^_i . S_j/|S_j|) = 1 - |S_j| / n_j`` because the
    members' unit keys sum to ``S_j``.  It lies in [0, 1]; NaN for an empty
    cluster.
    """
    S = np.asarray(S, np.float64)
    n = np.asarray(n, np.int64)
    out = np.full(len(n), np.nan)
    nz = n > 0
    out[nz] = 1.0 - np.sqrt(np.sum(S[nz] * S[nz], axis=1)) / n[nz]
    return out


def split(state: dict, x: np.ndarray, threshold: float, round_bf16: bool = True) -> dict:
    """Drift-triggered split (ClusterKV article §3.2: a cluster whose mean
    intra-cluster distance exceeds a threshold is split).

    ``state`` holds ``assign`` (labels of the clustered keys ``x`` [m, d], in
    token order), ``cdir``, ``csum`` and ``csize``; the number of clusters
    stays ``K`` (the slot count).  Readings taken where the article is silent:

    * drift is ``drift(S, n)``; a cluster is a candidate when it has at least
      two members and its drift is strictly above ``threshold``;
    * a split needs an empty slot (``n_f = 0``: a reserved slot, or a cluster
      that K-means left empty).  Candidates in decreasing drift (ties: smaller
      index) are paired with the empty slots in increasing index, as far as the
      slots go;
    * splitting ``j`` into ``f``: the seed is the member whose cosine to the
      current direction ``c~_j`` is smallest (ties: earliest token); ``f``
      gets the direction ``bf16(x^_seed)``; every member of ``j`` then takes
      the cosine argmax between ``c~_j`` and that seed direction (ties: the
      smaller slot index).  One such round, members of other clusters are not
      moved;
    * afterwards the sums, sizes and directions of every cluster are those of
      the new labels (an empty cluster keeps its previous direction).

    Cosines and scores are float64 dot products of bfloat16 values (exact
    products); the decisions are taken on those values.  Returns the new
    state plus ``pairs`` [(j, f)] and ``seeds`` (token-order index of each
    pair's seed).
    """
    x = np.asarray(x, np.float64)
    a = np.asarray(state["assign"], np.int64).copy()
    c = np.asarray(state["cdir"], np.float64)
    n = np.asarray(state["csize"], np.int64)
    k = c.shape[0]
    dr = drift(state["csum"], n)
    cands = [j for j in range(k) if n[j] >= 2 and dr[j] > threshold]
    cands.sort(key=lambda j: (-dr[j], j))
    free = [j for j in range(k) if n[j] == 0]
    pairs = list(zip(cands, free))
    seeds = []
    norms = np.sqrt(np.sum(x * x, axis=1))
    for j, f in pairs:
        members = np.flatnonzero(a == j)
        xm = x[members]
        cos = np.zeros(len(members))
        nz = norms[members] > 0
        cos[nz] = (xm[nz] @ c[j]) / norms[members][nz]
        seed = int(members[int(np.argmin(cos))])
        seeds.append(seed)
        cf = normalise(x[seed:seed + 1])[0]
        if round_bf16:
            cf = bf16.round_value(cf)
        lo, hi = (j, f) if j < f else (f, j)
        two = np.stack([c[lo], cf] if lo == j else [cf, c[hi]])
        pick = np.argmax(xm @ two.T, axis=1)
        a[members] = np.where(pick == 0, lo, hi)
    S, M, n_new = unit_sums(x, a, k)
    c_new = directions(S, n_new, c, round_bf16)
    return dict(assign=a, cdir=c_new, csum=S, msum=M, csize=n_new, pairs=pairs, seeds=seeds, drift=dr)
