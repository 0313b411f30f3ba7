"""bench.py's contract pieces that need no GPU: the multi-GPU refusal and the
algorithmic byte counts its roofline is priced on."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_bytes_of_the_benchmark_launch():
    # 64 units x ((16 sinks + 2048 recalled + 22 recent) rows x 512 B + 2048 x 4 B indices
    # + 4 x 128 x 2 B queries + 4 x 128 x 4 B outputs)
    per_unit = (16 + 2048 + 22) * 512 + 2048 * 4 + 4 * 128 * 2 + 4 * 128 * 4
    assert per_unit == 1_079_296
    assert bench.decode_bytes(64, 16, 2048, 22, 4) == 64 * per_unit == 69_074_944


def test_select_and_incremental_bytes():
    # select: mu (K x 128 x 4 B), sizes and offsets, q, the cut cluster's keys and perm, positions
    assert bench.select_bytes(1, 400, 2048, 4, 82) == 4 * 400 * 128 + 8 * 400 + 4 + 2 * 4 * 128 + 82 * 260 + 4 * 2048
    # incremental: every clustered token's K and V gathered and written dominates
    b = bench.incremental_bytes(128, 400, 32752, 320)
    rows = 128 * (32752 + 320) * 4 * 256
    assert rows < b < 1.1 * rows


def test_split_bytes():
    # split: per split-cluster row the key once plus token id and label; the rebuild
    # (norms, counting sort, K and V gathered and written in cluster order) dominates
    units, K, m, rows = 128, 416, 33072, 284019
    b = bench.split_bytes(units, K, m, rows)
    d = 128
    per_cluster = 8 * d + 4 + 2 * 2 * d + 2 * 8 * d + 4 * d + 4 * 2 + 4
    assert b == units * (K * per_cluster + m * (12 + 8 * d)) + rows * (2 * d + 8)
    gather = units * m * 4 * 2 * d
    assert gather < b < 1.1 * gather


def test_assign_flops_of_the_benchmark_launch():
    # one layer of the Llama-shaped stack: 64 units x 32752 keys x 400 directions x 128 dims x 2
    assert bench.assign_flops(64, 32752, 400) == 2 * 64 * 32752 * 400 * 128 == 214_643_507_200
