"""The benchmark's own accounting, on the CPU.

bench.py reports algorithmic TFLOP/s from its count of visible (query, key)
pairs, and algorithmic bytes from its count of stored dS tiles; both are
checked here against the oracle's token positions (oracle/ring.py), by brute
force on small rings and by the closed form for the full causal workloads.
The refusal of a multi-GPU run is checked too (it must not need a GPU).
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import ring

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LAYOUTS = ("contiguous", "striped", "zigzag")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P,Bb", [(1, 6), (3, 10), (4, 8), (5, 12), (8, 16)])
def test_pair_count_matches_the_oracle_per_rank(layout, causal, P, Bb):
    per_rank = ring.unmasked_pairs_per_rank(layout, P, Bb, causal)
    for i in range(P):
        assert bench.pair_count(layout, causal, P, Bb, [i]) == per_rank[i], (layout, causal, P, Bb, i)
    assert bench.pair_count(layout, causal, P, Bb, range(P)) == sum(per_rank)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_pair_count_of_the_whole_causal_ring_is_the_triangle(layout):
    """Over all ranks every layout covers each causal pair once: L (L + 1) / 2
    per head. The workload-5 figure (32 heads, 32768 tokens, ring of 8) is
    17,180,393,472 pairs, and the 65536-token ring of 16 follows too."""
    for P, Bb in ((8, 4096), (16, 4096), (4, 6)):
        L = P * Bb
        assert bench.pair_count(layout, True, P, Bb, range(P)) == L * (L + 1) // 2
    assert 32 * bench.pair_count("striped", True, 8, 4096, range(8)) == 17_180_393_472


def _brute_key_extent(layout, i, j, Bb, P, a):
    """Keys of block j that local row a of block i sees, from token positions."""
    tq = ring.token_position(layout, P, Bb, i, a)
    tk = ring.token_position(layout, P, Bb, j, np.arange(Bb))
    vis = ring.pair_visible(tq, tk, True)
    n = int(vis.sum())
    # visible keys form a prefix of the block in every layout (positions ascend)
    assert vis[:n].all() and not vis[n:].any()
    return n


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("P,Bb", [(3, 10), (4, 200), (5, 130)])
def test_key_extent_and_stored_ds_tiles_from_token_positions(layout, P, Bb):
    if layout == "zigzag" and Bb % 2:
        pytest.skip("zigzag needs an even block length")
    tiles = 0
    for i in range(P):
        for j in range(P):
            for a in range(Bb):
                e = _brute_key_extent(layout, i, j, Bb, P, a)
                assert bench.key_extent(layout, True, i, j, Bb, a) == e
            for qt in range(math.ceil(Bb / 64)):
                last = min(64 * qt + 63, Bb - 1)
                tiles += math.ceil(_brute_key_extent(layout, i, j, Bb, P, last) / 128)
    assert bench.stored_ds_tiles(layout, True, P, Bb, range(P)) == tiles


def test_more_than_one_gpu_is_refused_without_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
