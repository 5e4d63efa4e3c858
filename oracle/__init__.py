"""CPU oracle for exact blockwise (ring) attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy implementations of what the GPU path computes,
written from the pages that describe the method (cited per function). Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path (the HIP library and its binding)
never does, and shares no code with it.

Modules:
  attention -- full-softmax attention forward/backward (the definition,
               with K/V heads optionally shared by groups of query heads),
               the log-sum-exp merge of two partial results, and the pages'
               online-softmax loop run in ring order (for self-checks).
  ring      -- ring schedule, token layouts (contiguous / striped / zigzag), block
               classification, per-device work counts and the pages' tick
               simulation.
  bpt       -- a Blockwise Parallel Transformer layer: per query block,
               attention, output projection, residual + layer norm,
               feedforward network, residual + layer norm.

Every function here is pinned by a CPU test (brute force, closed forms,
library routines, the invariants the pages state, or values the pages print).
"""
from .attention import (  # noqa: F401
    attention_fwd,
    attention_bwd,
    attention_bwd_sampled,
    merge_lse,
    blockwise_ring_fwd,
    NEG_INF,
)
from .ring import (  # noqa: F401
    ring_schedule,
    layout_perm,
    token_position,
    block_relation,
    pair_visible,
    unmasked_pairs_per_rank,
    block_visits,
    tick_schedule,
)
from . import bpt  # noqa: F401,E402
