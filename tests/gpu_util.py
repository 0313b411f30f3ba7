"""Helpers for the GPU parity tests: host<->device bf16 moves and tolerance logic.

Inputs always come from ``synth`` (or from the oracle, for teacher-forced
state); GPU outputs are only ever compared, never fed to the oracle.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import bf16

DECODE_ATOL = 2e-3        # max |GPU f32 - oracle f64| of a decode output element
ASSIGN_MARGIN = 1e-4      # relative top-2 margin below which an assignment may differ
SELECT_GAP = 1e-4         # relative score gap below which a recall boundary may differ
MISMATCH_FRACTION = 1e-3  # overall allowed fraction of differing labels / recalled tokens


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def assign_margins(x: np.ndarray, cdir: np.ndarray) -> np.ndarray:
    """Relative top-2 margin (s1 - s2) / |x| of every key against the directions."""
    s = x @ cdir.T
    if s.shape[1] == 1:
        return np.full(s.shape[0], np.inf)
    part = np.partition(s, -2, axis=1)
    norms = np.linalg.norm(x, axis=1)
    norms[norms == 0] = 1.0
    return (part[:, -1] - part[:, -2]) / norms


def compare_assign(gpu: np.ndarray, ora: np.ndarray, x: np.ndarray, cdir: np.ndarray):
    """(mismatches, unexcused) where an excused key has a top-2 margin <= ASSIGN_MARGIN."""
    diff = np.nonzero(np.asarray(gpu) != np.asarray(ora))[0]
    if len(diff) == 0:
        return 0, 0
    marg = assign_margins(x[diff], cdir)
    return len(diff), int(np.sum(marg > ASSIGN_MARGIN))


def selection_boundary_gap(sel: dict, k_clu_vals: np.ndarray, offsets: np.ndarray) -> float:
    """Smallest relative score gap across the oracle's recall boundaries.

    Cluster level: between the last whole cluster, the cut cluster and the next
    one in visit order.  Token level: between the last taken and first untaken
    token of the cut cluster.  A GPU selection that differs from the oracle's is
    excused when this gap is <= SELECT_GAP.
    """
    s = sel["scores"]
    order = sel["order"]
    taken_ranks = []
    # rank of the cut cluster in visit order (or the end)
    if sel["cut"] >= 0:
        rc = int(np.nonzero(order == sel["cut"])[0][0])
        taken_ranks = [rc - 1, rc]
    gaps = [math.inf]
    for r in taken_ranks:
        if 0 <= r and r + 1 < len(order):
            a, b = s[order[r]], s[order[r + 1]]
            if np.isfinite(a) and np.isfinite(b):
                gaps.append(abs(a - b) / max(1.0, abs(a)))
    if sel["cut"] >= 0 and sel["need"] > 0:
        lo, hi = int(offsets[sel["cut"]]), int(offsets[sel["cut"] + 1])
        ts = np.sort(k_clu_vals[lo:hi] @ sel["q_bar"])[::-1]
        need = sel["need"]
        if need < len(ts):
            gaps.append(abs(ts[need - 1] - ts[need]) / max(1.0, abs(ts[need - 1])))
    return min(gaps)


def widen(bits):
    return bf16.widen(bits)
