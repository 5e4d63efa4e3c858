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


def block_visits(owner, P: int, block_len: int) -> list:
    """Per-device total of causal KV-block visits, the chapter's balance
    measure ("Worked Demo: A 4-Device Ring in Discrete Ticks"): with the
    sequence cut into contiguous blocks of ``block_len`` rows, row r attends
    keys of blocks 0 .. floor(r / block_len), which is floor(r / block_len) + 1
    block visits, and those visits count for the device that owns row r.
    ``owner[r]`` is that device (r // block_len for the contiguous layout,
    r mod P for the striped one). Device totals are a weighted histogram of
    the owners.
    """
    owner = np.asarray(owner, dtype=np.int64)
    visits = np.arange(owner.size) // block_len + 1
    return [int(x) for x in np.bincount(owner, weights=visits, minlength=P)]


def tick_schedule(P: int, compute_ticks: int, hop_ticks: int, overlapped: bool) -> dict:
    """Device 0's ring steps in the chapter's tick model ("Ring Attention:
    Compute While You Communicate", and the discrete-tick demo that follows
    it): every step computes one block attention (c = compute_ticks) and
    passes one KV block to the next device (m = hop_ticks). Run one after
    the other a step occupies c + m ticks, the hop starting as the compute
    ends; with the hop issued at the start of the step and run alongside the
    compute, a step occupies max(c, m) ticks, so the whole ring takes
    P * max(c, m) instead of P * (c + m) (all of the hop hidden when m <= c).

    Returns, for steps k = 0 .. P-1: "compute" [P, 2] and "hop" [P, 2] tick
    intervals [start, end), "block" (the KV block device 0 holds at step k,
    (0 - k) mod P), and "total" (the tick at which the ring is done).
    """
    period = max(compute_ticks, hop_ticks) if overlapped else compute_ticks + hop_ticks
    start = np.arange(P, dtype=np.int64) * period
    hop_start = start if overlapped else start + compute_ticks
    return {
        "compute": np.stack([start, start + compute_ticks], axis=1),
        "hop": np.stack([hop_start, hop_start + hop_ticks], axis=1),
        "block": (-np.arange(P)) % P,
        "total": int(P * period),
    }
