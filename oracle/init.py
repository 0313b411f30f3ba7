"""Seeded initial centroid indices of the prefill clustering, one unit at a time.

Test infrastructure only (see ``oracle/__init__``).

The ClusterKV article (§3.2, prefill) clusters the keys by K-means but does not
say how the initial centroids are picked.  Reading taken: K distinct key
indices drawn uniformly without replacement by Floyd's sampling algorithm
(Bentley and Floyd, "A sample of brilliance", CACM 1987), driven by the
SplitMix64 generator (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) with state ``seed + unit``.  The centroid
with index j starts at the j-th index the sampler inserts.

Floyd's algorithm, as used here: for j = m - K, ..., m - 1, draw a 64-bit
r, let t = r mod (j + 1); insert t if it is not yet in the sample, else insert
j.  Every K-subset of [0, m) is equally likely (up to the negligible bias of
the modulo), and the draw needs exactly K generator outputs.
"""

from __future__ import annotations

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(state: int):
    """Infinite stream of SplitMix64 outputs from the given 64-bit state.

    Each step adds the golden-ratio increment to the state, then mixes it:
    xor-shift by 30, multiply by 0xBF58476D1CE4E5B9, xor-shift by 27, multiply
    by 0x94D049BB133111EB, xor-shift by 31 (all modulo 2^64).
    """
    x = state & MASK64
    while True:
        x = (x + GOLDEN_GAMMA) & MASK64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        yield z ^ (z >> 31)


def floyd_sample(m: int, k: int, draws) -> list[int]:
    """K distinct indices in [0, m) from Floyd's algorithm, in insertion order.

    ``draws`` yields the 64-bit random numbers, one per inserted index.
    """
    if not (0 <= k <= m):
        raise ValueError("need 0 <= K <= m")
    chosen: list[int] = []
    present: set[int] = set()
    for j in range(m - k, m):
        t = next(draws) % (j + 1)
        pick = t if t not in present else j
        present.add(pick)
        chosen.append(pick)
    return chosen


def init_indices(seed: int, unit: int, m: int, k: int) -> list[int]:
    """The initial centroid indices of one unit: Floyd driven by SplitMix64 from ``seed + unit``."""
    return floyd_sample(m, k, splitmix64((seed + unit) & MASK64))
