"""The host/device schedule header (ring order, token layouts, causal block
relations, pair counts) compiled with g++ and checked against the oracle's
independent Python versions and brute force over token positions."""
import itertools
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_blockwise_attention_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "ra_schedule.h"
int main() {
  using namespace ra;
  // ring order
  for (int P = 1; P <= 9; ++P)
    for (int i = 0; i < P; ++i) {
      printf("ring %d %d", P, i);
      for (int k = 0; k < P; ++k) printf(" %d", ring_block(i, k, P));
      printf("\n");
      for (int k = 0; k < P; ++k)
        if (ring_block(ring_rank(ring_block(i, k, P), k, P), k, P) != ring_block(i, k, P) ||
            ring_rank(ring_block(i, k, P), k, P) != i) printf("BAD inverse %d %d %d\n", P, i, k);
    }
  // relations and pair counts
  const int Ps[] = {1, 2, 3, 5, 8};
  const long Bbs[] = {1, 3, 8, 13};
  const long BbsEven[] = {2, 4, 8, 14};
  for (int layout = 0; layout < 3; ++layout)
    for (int causal = 0; causal < 2; ++causal)
      for (int P : Ps)
        for (int bi = 0; bi < 4; ++bi) {
          const long Bb = layout == 2 ? BbsEven[bi] : Bbs[bi];
          for (int i = 0; i < P; ++i) {
            for (int j = 0; j < P; ++j) {
              BlockRel r = block_relation(layout, causal, i, j, (int)Bb);
              printf("rel %d %d %d %ld %d %d %d", layout, causal, P, Bb, i, j, r.kind);
              for (long a = 0; a < Bb; ++a) printf(" %ld", (long)row_extent(r, a));
              printf(" |");
              for (long ahi = 0; ahi < Bb; ++ahi) printf(" %ld", (long)visible_key_extent(r, ahi, Bb));
              printf(" |");
              for (long b = 0; b < Bb; ++b) printf(" %ld", (long)first_row_seeing(r, b, Bb));
              printf(" | %ld\n", (long)visible_pairs(r, 0, Bb - 1, Bb));
            }
            printf("pairs %d %d %d %ld %d %ld\n", layout, causal, P, Bb, i, (long)rank_pairs(layout, causal, P, Bb, i));
          }
        }
  for (int layout = 0; layout < 3; ++layout)
    for (int s = 0; s < 3; ++s)
      for (long x = 0; x < 6; ++x)
        printf("pos %d %d %ld %ld\n", layout, s, x, (long)token_position(layout, 3, 6, s, x));
  return 0;
}
"""


@pytest.fixture(scope="module")
def schedule_output(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("sched")
    src = d / "t.cpp"
    src.write_text(DRIVER)
    exe = d / "t"
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines()


LAYOUT_NAMES = {0: "contiguous", 1: "striped", 2: "zigzag"}


def test_ring_order(schedule_output):
    rows = [l.split() for l in schedule_output if l.startswith("ring ")]
    assert rows and not any(l.startswith("BAD") for l in schedule_output)
    for r in rows:
        P, i = int(r[1]), int(r[2])
        assert [int(x) for x in r[3:]] == oracle.ring_schedule(P, i)


def test_block_relations_against_brute_force(schedule_output):
    rows = [l for l in schedule_output if l.startswith("rel ")]
    assert len(rows) > 100
    for line in rows:
        head, hi_s, first_s, pairs = line.split("|")
        f = head.split()
        layout, causal, P, Bb, i, j, kind = (int(x) for x in f[1:8])
        row_ext = [int(x) for x in f[8:]]
        extents = [int(x) for x in hi_s.split()]
        first = [int(x) for x in first_s.split()]
        name = LAYOUT_NAMES[layout]
        a = np.arange(Bb)[:, None]
        b = np.arange(Bb)[None, :]
        tq = oracle.token_position(name, P, Bb, i, a)
        tk = oracle.token_position(name, P, Bb, j, b)
        vis = oracle.pair_visible(tq, tk, bool(causal))
        assert int(pairs) == int(vis.sum())
        # the exact mask: row a sees the keys 0 .. ext(a) - 1 and no other
        assert np.array_equal(vis, b < np.array(row_ext)[:, None]), (layout, causal, P, Bb, i, j)
        # extent: number of leading keys that rows 0..ahi can see, and nothing beyond it
        for ahi, ext in enumerate(extents):
            seen = vis[: ahi + 1].any(axis=0)
            assert not seen[ext:].any()
            if ext:
                assert seen[ext - 1]
        # first row that sees each key
        for key in range(Bb):
            rows_seeing = np.flatnonzero(vis[:, key])
            assert first[key] == (int(rows_seeing[0]) if rows_seeing.size else Bb)
        if kind == 0:
            assert not vis.any()
        elif kind == 1:
            assert vis.all()


def test_rank_pairs_match_oracle(schedule_output):
    rows = [l.split() for l in schedule_output if l.startswith("pairs ")]
    assert rows
    cache = {}
    for r in rows:
        layout, causal, P, Bb, i, pairs = (int(x) for x in r[1:])
        key = (layout, causal, P, Bb)
        if key not in cache:
            cache[key] = oracle.unmasked_pairs_per_rank(LAYOUT_NAMES[layout], P, Bb, causal=bool(causal))
        assert pairs == cache[key][i]


def test_token_positions(schedule_output):
    for r in (l.split() for l in schedule_output if l.startswith("pos ")):
        layout, s, x, t = (int(v) for v in r[1:])
        assert t == int(oracle.token_position(LAYOUT_NAMES[layout], 3, 6, s, x))
