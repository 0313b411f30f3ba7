"""Host-side seeded generators for the ClusterKV workloads.

Recipe (the same for every workload; sizes come from ``CONFIGS``):

* every unit (one KV head of one sequence of one layer) owns ``components``
  mixture centres ``8 * g / |g|`` with ``g ~ N(0, I_128)``;
* a key is ``centre[z] + N(0, sigma^2 I)`` with ``z`` uniform over the
  components and ``sigma = 1``; the first 16 (sink) keys come from the same
  mixture;
* a value is ``N(0, I)``;
* a query of unit ``u`` is ``centre_u[z_q] + N(0, I)`` with ``z_q`` uniform;
* everything is drawn in float64 and stored as bfloat16 bit patterns
  (``uint16``), rounded to nearest-even through float32.

Each unit has its own PCG64 stream seeded with ``[seed, unit]`` so any unit can
be regenerated alone.  Nothing here belongs to the method: the draws are the
inputs, and the initial centroid indices are random draws handed to both the
GPU path and the oracle.
"""

from __future__ import annotations

import dataclasses

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    layers: int
    batch: int
    n_kv_heads: int
    group: int            # query heads per KV head (GQA group)
    n_tokens: int         # tokens already clustered (sinks included)
    n_recent: int         # unclustered recent tokens on top of n_tokens
    n_sink: int
    n_clusters: int
    iters: int
    budget: int
    components: int
    steps: int            # decode steps in the workload
    new_tokens: int = 0   # tokens appended before an incremental pass
    new_components: int = 0
    new_fraction: float = 0.0
    seed_base: int = 0    # data seed = 1000 + seed_base, init 2000 + ..., query 3000 + ...

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def m(self) -> int:
        return self.n_tokens - self.n_sink

    @property
    def data_seed(self) -> int:
        return 1000 + self.seed_base

    @property
    def init_seed(self) -> int:
        return 2000 + self.seed_base

    @property
    def query_seed(self) -> int:
        return 3000 + self.seed_base


CONFIGS = {
    # single head, 2k context, 32-component mixture, 24 clusters, budget 256
    "single-head-2k": WorkloadConfig(
        name="single-head-2k", layers=1, batch=1, n_kv_heads=1, group=1,
        n_tokens=2048, n_recent=0, n_sink=16, n_clusters=24, iters=10,
        budget=256, components=32, steps=1, seed_base=0),
    # one Llama-3.1-8B-shaped layer: 8 KV heads x 4 query heads, 32k context
    "llama8b-layer-32k": WorkloadConfig(
        name="llama8b-layer-32k", layers=1, batch=1, n_kv_heads=8, group=4,
        n_tokens=32768, n_recent=0, n_sink=16, n_clusters=400, iters=10,
        budget=1024, components=512, steps=1, seed_base=1),
    # 32 such layers, batch 8, budget 2048, 20 decode steps
    "llama8b-stack-32k-b8": WorkloadConfig(
        name="llama8b-stack-32k-b8", layers=32, batch=8, n_kv_heads=8, group=4,
        n_tokens=32768, n_recent=0, n_sink=16, n_clusters=400, iters=10,
        budget=2048, components=512, steps=20, seed_base=2),
    # incremental clustering on the Llama layer shape, batch 16, +320 keys
    "llama8b-incremental-b16": WorkloadConfig(
        name="llama8b-incremental-b16", layers=1, batch=16, n_kv_heads=8,
        group=4, n_tokens=32768, n_recent=0, n_sink=16, n_clusters=400,
        iters=10, budget=1024, components=512, steps=1, new_tokens=320,
        new_components=8, new_fraction=0.1, seed_base=3),
    # GLM4-9B-like stack: 40 layers, 32 query heads over 2 KV heads, batch 16
    "glm4-stack-32k-b16": WorkloadConfig(
        name="glm4-stack-32k-b16", layers=40, batch=16, n_kv_heads=2, group=16,
        n_tokens=32468, n_recent=300, n_sink=16, n_clusters=410, iters=10,
        budget=2048, components=512, steps=50, new_tokens=320, seed_base=4),
}


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 data to bfloat16 bit patterns (via float32, nearest-even)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _centres(rng: np.random.Generator, count: int, d: int, radius: float) -> np.ndarray:
    g = rng.standard_normal((count, d))
    return radius * g / np.linalg.norm(g, axis=1, keepdims=True)


def make_unit_inputs(seed: int, unit: int, n_tokens: int, components: int,
                     d: int = HEAD_DIM, radius: float = 8.0, sigma: float = 1.0,
                     capacity: int | None = None):
    """Keys, values and centres of one unit.

    Returns ``(k_bits, v_bits, centres)`` with ``k_bits``/``v_bits`` uint16
    ``[capacity, d]`` (rows past ``n_tokens`` are zero) and ``centres``
    float64 ``[components, d]``.
    """
    capacity = n_tokens if capacity is None else capacity
    rng = np.random.default_rng([seed, unit])
    centres = _centres(rng, components, d, radius)
    z = rng.integers(0, components, size=n_tokens)
    k = centres[z] + sigma * rng.standard_normal((n_tokens, d))
    v = rng.standard_normal((n_tokens, d))
    kb = np.zeros((capacity, d), np.uint16)
    vb = np.zeros((capacity, d), np.uint16)
    kb[:n_tokens] = f64_to_bf16_bits(k)
    vb[:n_tokens] = f64_to_bf16_bits(v)
    return kb, vb, centres


def make_layer_inputs(cfg: WorkloadConfig, layer: int = 0, capacity: int | None = None,
                      units: list[int] | None = None):
    """Keys/values/centres for the units of one layer (all units by default).

    Returns ``(k [U, capacity, d] uint16, v [...], centres [U, C, d])``.
    ``n_tokens + n_recent`` rows are filled.
    """
    n = cfg.n_tokens + cfg.n_recent
    capacity = n if capacity is None else capacity
    units = list(range(cfg.units)) if units is None else units
    ks, vs, cs = [], [], []
    for u in units:
        kb, vb, c = make_unit_inputs(cfg.data_seed, layer * cfg.units + u, n,
                                     cfg.components, capacity=capacity)
        ks.append(kb)
        vs.append(vb)
        cs.append(c)
    return np.stack(ks), np.stack(vs), np.stack(cs)


def make_queries(seed: int, centres: np.ndarray, group: int, step: int = 0,
                 unit_ids: list[int] | None = None, d: int = HEAD_DIM) -> np.ndarray:
    """One query per query head: ``[U, group, d]`` uint16 bf16 bits.

    ``centres`` is ``[U, C, d]``; each query head picks a centre uniformly.
    """
    U = centres.shape[0]
    unit_ids = list(range(U)) if unit_ids is None else unit_ids
    out = np.empty((U, group, d), np.uint16)
    for i, u in enumerate(unit_ids):
        rng = np.random.default_rng([seed, step, u])
        z = rng.integers(0, centres.shape[1], size=group)
        q = centres[i][z] + rng.standard_normal((group, d))
        out[i] = f64_to_bf16_bits(q)
    return out


def make_init_indices(seed: int, units: int, m: int, k: int,
                      unit_ids: list[int] | None = None) -> np.ndarray:
    """``k`` distinct random indices in ``[0, m)`` per unit, ``[units, k]`` int32.

    These are the random draws that pick the initial centroids; the GPU path
    and the oracle both take them as inputs.
    """
    unit_ids = list(range(units)) if unit_ids is None else unit_ids
    out = np.empty((len(unit_ids), k), np.int32)
    for i, u in enumerate(unit_ids):
        rng = np.random.default_rng([seed, u])
        out[i] = rng.choice(m, size=k, replace=False).astype(np.int32)
    return out


def make_new_tokens(seed: int, centres: np.ndarray, count: int, new_components: int,
                    new_fraction: float, unit_ids: list[int] | None = None,
                    d: int = HEAD_DIM, radius: float = 8.0, sigma: float = 1.0):
    """Keys/values appended before an incremental pass.

    ``round(count * new_fraction)`` keys come from ``new_components`` fresh
    centres, the rest from the unit's own mixture; their positions are
    shuffled.  Returns ``(k [U, count, d], v [U, count, d], new_centres
    [U, new_components, d])``.
    """
    U = centres.shape[0]
    unit_ids = list(range(U)) if unit_ids is None else unit_ids
    n_new = int(round(count * new_fraction))
    ks = np.empty((U, count, d), np.uint16)
    vs = np.empty((U, count, d), np.uint16)
    nc = np.zeros((U, max(new_components, 0), d))
    for i, u in enumerate(unit_ids):
        rng = np.random.default_rng([seed, 7, u])
        if new_components > 0:
            nc[i] = _centres(rng, new_components, d, radius)
        z_old = rng.integers(0, centres.shape[1], size=count - n_new)
        rows = [centres[i][z_old]]
        if n_new:
            z_new = rng.integers(0, new_components, size=n_new)
            rows.append(nc[i][z_new])
        mu = np.concatenate(rows, axis=0)
        mu = mu[rng.permutation(count)]
        k = mu + sigma * rng.standard_normal((count, d))
        v = rng.standard_normal((count, d))
        ks[i] = f64_to_bf16_bits(k)
        vs[i] = f64_to_bf16_bits(v)
    return ks, vs, nc


def make_planted_groups(seed: int, sizes: list[int], n_sink: int = 16, d: int = HEAD_DIM,
                        radius: float = 8.0, sigma: float = 1.0, extra_rows: int = 0):
    """One unit whose clustered keys form well separated groups of the given sizes.

    Group ``g`` has centre ``radius * c_g`` with ``c_g`` a random unit vector;
    its keys are ``centre + N(0, sigma^2 I)``.  The ``n_sink`` sink keys and
    ``extra_rows`` rows after the clustered ones come from the groups too.  The
    clustered tokens' group labels are shuffled over token order.  Returns
    ``(k_bits [n, d], v_bits [n, d], centres [G, d], labels [m])`` with
    ``n = n_sink + sum(sizes) + extra_rows`` and ``labels`` the group of
    clustered token ``i`` (token id ``n_sink + i``).
    """
    rng = np.random.default_rng([seed, 11])
    centres = _centres(rng, len(sizes), d, radius)
    labels = np.concatenate([np.full(sz, g, np.int64) for g, sz in enumerate(sizes)])
    labels = labels[rng.permutation(len(labels))]
    z_sink = rng.integers(0, len(sizes), size=n_sink)
    z_extra = rng.integers(0, len(sizes), size=extra_rows)
    z = np.concatenate([z_sink, labels, z_extra])
    k = centres[z] + sigma * rng.standard_normal((len(z), d))
    v = rng.standard_normal((len(z), d))
    return f64_to_bf16_bits(k), f64_to_bf16_bits(v), centres, labels
