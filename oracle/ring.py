"""Ring schedule, token layouts, causal block relations and work counts.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain Python/numpy.

Notation: P devices (ring size), sequence of L = P * Bb tokens, Bb tokens per
block. Device i keeps query block i; at ring step k it holds KV block
j = (i - k) mod P.

Sources (page title, section):
  * "Ring Attention: Sequence Parallelism for Long Context" (book chapter),
    sections "Ring Attention: Compute While You Communicate" (ring diagram:
    step k attends KV block (i - k) mod P; device 0 sees KV[0], KV[3], KV[2],
    KV[1]), "The Causal-Mask Problem: Striped Attention" (row r goes to device
    r mod P; the zigzag variant's two symmetric half-blocks) and "Worked Demo: A 4-Device Ring in Discrete Ticks" (tick model
    and the per-device work metric).
  * "Ring Attention 論文分析" (blog), sections "リングトポロジーと KV の循環"
    (send to rank+1, receive from rank-1), "リング通信パターン" (N=4 step
    table) and "Causal Masking の処理" (skip / diagonal mask / full).
"""
from __future__ import annotations

import numpy as np


def ring_schedule(P: int, i: int) -> list:
    """KV block held by device ``i`` at each step k = 0..P-1: (i - k) mod P.

    Each device forwards its KV block to (i + 1) mod P and receives from
    (i - 1) mod P, so after k hops device i holds the block that started on
    device i - k. Step 0 is the device's own block.
    """
    if P < 1 or not (0 <= i < P):
        raise ValueError("need P >= 1 and 0 <= i < P")
    return [(i - k) % P for k in range(P)]


def token_position(layout: str, P: int, block_len: int, block, local):
    """Original token index of local row ``local`` of block ``block``.

    contiguous: device s owns tokens s*Bb .. (s+1)*Bb - 1, in order.
    striped:    token t goes to device t mod P; within a device the rows keep
                ascending token order, so local row x of block s is token
                x*P + s (the pages fix only the device of each row; ascending
                order inside a device is the plain reading).
    zigzag:     each device holds two half-blocks placed symmetrically near the
                start and the end of the sequence: with the sequence cut into
                2P chunks of Bb/2 tokens, device s holds chunk s and chunk
                2P-1-s. The plain reading of the order: chunk s first, each
                chunk in ascending token order (needs Bb even).
    Works elementwise on numpy integer arrays.
    """
    if layout == "contiguous":
        return np.asarray(block) * block_len + np.asarray(local)
    if layout == "striped":
        return np.asarray(local) * P + np.asarray(block)
    if layout == "zigzag":
        if block_len % 2:
            raise ValueError("zigzag needs an even block length")
        half = block_len // 2
        block, local = np.asarray(block), np.asarray(local)
        first = block * half + local
        second = (2 * P - 1 - block) * half + (local - half)
        return np.where(local < half, first, second)
    raise ValueError(f"unknown layout {layout!r}")


def layout_perm(L: int, P: int, layout: str) -> np.ndarray:
    """Blocked -> original index map: perm[s*Bb + x] = token_position(s, x).

    ``x[:, perm]`` gathers an original-order [B, L, ...] tensor into blocked
    order (block 0 rows first); ``y[:, argsort(perm)]`` undoes it.
    """
    if L % P:
        raise ValueError("sequence length must split into P equal blocks")
    Bb = L // P
    s = np.repeat(np.arange(P), Bb)
    x = np.tile(np.arange(Bb), P)
    return token_position(layout, P, Bb, s, x).astype(np.int64)


def pair_visible(t_query, t_key, causal: bool):
    """Causal rule: key token t' is visible to query token t iff t' <= t."""
    if not causal:
        return np.ones(np.broadcast(np.asarray(t_query), np.asarray(t_key)).shape, dtype=bool)
    return np.asarray(t_key) <= np.asarray(t_query)


def block_relation(layout: str, P: int, block_len: int, i: int, j: int, causal: bool = True):
    """How KV block j's keys relate to query block i's rows.

    Returns ("none"|"all"|"band"|"first_half"|"second_half_rows", c): for
    "band", key b is visible to query a iff b - a <= c (local indices); for
    "first_half" every query row sees exactly the keys b < c; for
    "second_half_rows" rows a >= c see every key and rows a < c none. Derived
    from the token positions:
      contiguous: j > i -> none (the whole block lies in the future and is
                  skipped), j == i -> band with c = 0 (the diagonal block,
                  strictly-upper triangle masked), j < i -> all;
      striped:    b*P + j <= a*P + i  <=>  b - a <= 0 if j <= i else -1;
      zigzag:     (h = Bb/2; block s holds chunks s and 2P-1-s) a key in the
                  first half lies in chunk j <= P-1, before chunk 2P-1-i of
                  the query's second half, and a key in the second half lies in
                  chunk 2P-1-j >= P, after chunk i of the query's first half.
                  So j == i -> band 0 (chunk pairs on the diagonal), j < i ->
                  first_half h, j > i -> second_half_rows h.
    """
    if not causal:
        return ("all", None)
    if layout == "contiguous":
        if j > i:
            return ("none", None)
        if j == i:
            return ("band", 0)
        return ("all", None)
    if layout == "striped":
        return ("band", 0 if j <= i else -1)
    if layout == "zigzag":
        half = block_len // 2
        if j == i:
            return ("band", 0)
        return ("first_half", half) if j < i else ("second_half_rows", half)
    raise ValueError(f"unknown layout {layout!r}")


def unmasked_pairs_per_rank(layout: str, P: int, block_len: int, causal: bool = True) -> list:
    """Exact number of visible (query, key) pairs each device computes.

    Counts, for every query row of device i and every KV block j, the keys of
    block j whose token position is <= the query's (all keys when not
    causal). Key positions inside a block are ascending in every layout, so a
    sorted search gives the per-row count.
    """
    Bb = block_len
    out = []
    local = np.arange(Bb)
    for i in range(P):
        tq = token_position(layout, P, Bb, i, local)
        total = 0
        for j in range(P):
            if not causal:
                total += Bb * Bb
                continue
            tk = token_position(layout, P, Bb, j, local)
            total += int(np.searchsorted(tk, tq, side="right").sum())
        out.append(total)
    return out


def block_visit_work(assignment, P: int, block_len: int) -> list:
    """The chapter's demo metric: unmasked contiguous KV-block visits.

    Row r of the sequence needs KV blocks 0 .. r // Bb under a causal mask
    (blocks of Bb consecutive rows), i.e. r // Bb + 1 visits; the count is
    added to the device that owns row r under ``assignment`` (a list mapping
    each row to its device). Reproduces the demo exactly as printed, for both
    assignments.
    """
    work = [0] * P
    for r, dev in enumerate(assignment):
        work[dev] += r // block_len + 1
    return work


def ring_timeline(c: int, m: int, P: int, overlap: bool):
    """Device 0's schedule in the chapter's discrete-tick model.

    Each of the P steps computes one block attention (c ticks) and forwards
    one KV block (m ticks). Without overlap the hop starts when the compute
    ends and the next step waits for both (c + m per step); with overlap the
    hop runs alongside the compute and a step lasts max(c, m).

    Returns (steps, total) with steps = [(k, (c0, c1), (m0, m1), block)],
    ``block`` being the KV block device 0 holds and forwards at step k,
    (0 - k) mod P. (The printed demo labels the hop "KV[(k+1) % P]"; that
    label does not change any tick count.)
    """
    steps, t = [], 0
    for k in range(P):
        block = (0 - k) % P
        if overlap:
            steps.append((k, (t, t + c), (t, t + m), block))
            t += max(c, m)
        else:
            steps.append((k, (t, t + c), (t + c, t + c + m), block))
            t += c + m
    return steps, t
