"""Full-softmax attention in float64 — TEST INFRASTRUCTURE ONLY.

The method (blockwise attention with online softmax, run over a ring of KV
blocks) reaches exactly the result of ordinary softmax attention, up to
rounding order ("Ring Attention 論文分析" (blog), section "ブロック単位の分割
戦略": the correction keeps the blockwise result equal to the full softmax;
"序列并行性和环注意力" (article): partial results combine exactly). So the
oracle is that definition written out, per (batch, head), over chunks of
query rows, with a library matrix product as the only building block.

Conventions (shared with the GPU path's documentation, not its code):
  * tensors are [B, L, H, d] in original token order;
  * scores are scaled before the softmax: S = scale * Q K^T, scale = 1/sqrt(d)
    by default (blog, the forward listings multiply the product by scale);
  * causal: key token t' is visible to query token t iff t' <= t, in original
    token positions (blog, section "Causal Masking の処理");
  * lse is the natural log of sum_t' exp(S[t, t']) over the visible keys, the
    statistic the backward recomputes probabilities from (blog, section
    "逆伝播での KV 再循環": P = exp(scores - lse)); a row with no visible key
    has lse = -inf and output 0 (it only arises for partial key sets);
  * backward (same section): D = rowsum(dO * O), dV = P^T dO, dP = dO V^T,
    dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q;
  * grouped-query attention: K and V may have fewer heads (Hk) than Q (H),
    H a multiple of Hk; query head h reads key/value head h // (H / Hk), so
    consecutive query heads share one K/V head, and the gradient of a K/V
    head is the sum over the query heads that read it (blog, section
    "比較分析: Ring Attention vs Sequence Parallelism vs Tensor Parallelism":
    ring attention is fully compatible with GQA/MQA, e.g. 8 K/V heads).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _kv_group(H, Hk):
    """Query heads per K/V head (1 for ordinary multi-head attention)."""
    if Hk < 1 or H % Hk:
        raise ValueError(f"{H} query heads cannot share {Hk} K/V heads evenly")
    return H // Hk


def _kv_head(h, H, Hk):
    """The K/V head that query head h reads: consecutive query heads share one."""
    return h // (H // Hk)


def _kv_groups_of(heads, H, Hk):
    """The K/V heads that the query heads ``heads`` read, in order of first
    appearance; every query head that reads one of them must be in ``heads``."""
    groups = list(dict.fromkeys(_kv_head(h, H, Hk) for h in heads))
    if sorted(heads) != [h for h in range(H) if _kv_head(h, H, Hk) in groups]:
        raise ValueError("a gradient of shared K/V heads needs every query head of each group")
    return groups


def _positions(n, pos):
    return np.arange(n, dtype=np.int64) if pos is None else np.asarray(pos, dtype=np.int64)


def _scores(qc, kk, scale, tq, tk, causal):
    """Scaled scores of a chunk of query rows, masked entries -inf."""
    s = scale * (qc @ kk.T)
    if causal:
        s = np.where(tk[None, :] <= tq[:, None], s, NEG_INF)
    return s


def _softmax_stats(s):
    """Row max-shifted exponentials, their row sum and the row lse."""
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    ssum = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(ssum)
    return e, ssum, lse


def attention_fwd(q, k, v, causal, scale=None, q_pos=None, k_pos=None, heads=None, row_chunk=1024):
    """Softmax attention: returns (O [B, Lq, Hs, d], lse [B, Lq, Hs]).

    q: [B, Lq, H, d]; k, v: [B, Lk, Hk, d] (float64), Hk dividing H (query
    head h reads K/V head h // (H / Hk)). ``q_pos``/``k_pos`` give
    the original token position of each row (default 0..L-1); the causal mask
    is taken on those positions, so a row subset or a permuted sequence is
    computed by passing the rows with their positions. ``heads`` restricts the
    computation to a list of heads (outputs then hold only those).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Lq, H, d = q.shape
    Lk = k.shape[1]
    _kv_group(H, k.shape[2])
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    tq_all = _positions(Lq, q_pos)
    tk_all = _positions(Lk, k_pos)
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((B, Lq, len(heads), v.shape[3]))
    lse = np.zeros((B, Lq, len(heads)))
    for b in range(B):
        for hi, h in enumerate(heads):
            hk = _kv_head(h, H, k.shape[2])
            kk, vv = k[b, :, hk, :], v[b, :, hk, :]
            for r0 in range(0, Lq, row_chunk):
                r1 = min(Lq, r0 + row_chunk)
                tq = tq_all[r0:r1]
                if causal:
                    # keys later than every row of the chunk are masked for
                    # all of them; leaving them out changes no sum
                    keep = tk_all <= tq.max()
                    kc, vc, tk = kk[keep], vv[keep], tk_all[keep]
                else:
                    kc, vc, tk = kk, vv, tk_all
                if kc.shape[0] == 0:
                    o[b, r0:r1, hi] = 0.0
                    lse[b, r0:r1, hi] = NEG_INF
                    continue
                s = _scores(q[b, r0:r1, h, :], kc, scale, tq, tk, causal)
                e, ssum, l_ = _softmax_stats(s)
                with np.errstate(invalid="ignore", divide="ignore"):
                    out = (e @ vc) / ssum[:, None]
                out[ssum == 0] = 0.0
                o[b, r0:r1, hi] = out
                lse[b, r0:r1, hi] = l_
    return o, lse


def attention_bwd(q, k, v, do, causal, scale=None, heads=None, row_chunk=1024):
    """Gradients of sum(dO * O) for softmax attention over the whole sequence.

    Returns (dq, dk, dv, o, lse) for the selected query heads, float64:
    dq, o [B, L, Hs, d], lse [B, L, Hs]; dk, dv [B, L, Gs, d] for the Gs K/V
    heads those query heads read (with K/V heads shared, ``heads`` must hold
    whole groups). O and lse are the oracle's own.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, L, H, d = q.shape
    _kv_group(H, k.shape[2])
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = list(range(H)) if heads is None else list(heads)
    groups = _kv_groups_of(heads, H, k.shape[2])
    o, lse = attention_fwd(q, k, v, causal, scale=scale, heads=heads, row_chunk=row_chunk)
    t = np.arange(L, dtype=np.int64)
    dq = np.zeros((B, L, len(heads), d))
    dk = np.zeros((B, L, len(groups), d))
    dv = np.zeros((B, L, len(groups), v.shape[3]))
    for b in range(B):
        for hi, h in enumerate(heads):
            hk = _kv_head(h, H, k.shape[2])
            gi = groups.index(hk)
            kk, vv = k[b, :, hk, :], v[b, :, hk, :]
            for r0 in range(0, L, row_chunk):
                r1 = min(L, r0 + row_chunk)
                nk = r1 if causal else L  # keys beyond the chunk's last row are masked
                qc, doc, oc = q[b, r0:r1, h, :], do[b, r0:r1, h, :], o[b, r0:r1, hi, :]
                s = _scores(qc, kk[:nk], scale, t[r0:r1], t[:nk], causal)
                p = np.exp(s - lse[b, r0:r1, hi][:, None])
                dv[b, :nk, gi] += p.T @ doc
                dp = doc @ vv[:nk].T
                dd = (doc * oc).sum(axis=1)
                ds = _dsoftmax(p, dp, dd)
                dq[b, r0:r1, hi] = scale * (ds @ kk[:nk])
                dk[b, :nk, gi] += scale * (ds.T @ qc)
    return dq, dk, dv, o, lse


def attention_bwd_sampled(q, k, v, do, causal, q_rows, k_rows, scale=None, heads=None, row_chunk=1024):
    """dQ at query rows ``q_rows`` and dK, dV at key rows ``k_rows``.

    The same formulas as attention_bwd, evaluated only where asked: a row of
    dQ needs that query's scores against all keys; a row of dK / dV needs
    that key's column of probabilities over all queries, which needs every
    query's lse and D = rowsum(dO * O) (so the forward runs on all rows).
    Returns (dq [B, nq, Hs, d], dk [B, nk, Gs, d], dv [B, nk, Gs, d], o, lse),
    Gs the K/V heads read by the query heads ``heads`` (whole groups, as in
    attention_bwd).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, L, H, d = q.shape
    _kv_group(H, k.shape[2])
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = list(range(H)) if heads is None else list(heads)
    groups = _kv_groups_of(heads, H, k.shape[2])
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    o, lse = attention_fwd(q, k, v, causal, scale=scale, heads=heads, row_chunk=row_chunk)
    t = np.arange(L, dtype=np.int64)
    dq = np.zeros((B, len(q_rows), len(heads), d))
    dk = np.zeros((B, len(k_rows), len(groups), d))
    dv = np.zeros((B, len(k_rows), len(groups), v.shape[3]))
    for b in range(B):
        for hi, h in enumerate(heads):
            hk = _kv_head(h, H, k.shape[2])
            gi = groups.index(hk)
            qq, kk, vv, dd_o = q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h]
            dsum = (dd_o * o[b, :, hi]).sum(axis=1)
            lrow = lse[b, :, hi]
            for c0 in range(0, len(q_rows), row_chunk):
                rows = q_rows[c0:c0 + row_chunk]
                s = _scores(qq[rows], kk, scale, rows, t, causal)
                p = np.exp(s - lrow[rows][:, None])
                ds = _dsoftmax(p, dd_o[rows] @ vv.T, dsum[rows])
                dq[b, c0:c0 + len(rows), hi] = scale * (ds @ kk)
            for c0 in range(0, len(k_rows), row_chunk):
                cols = k_rows[c0:c0 + row_chunk]
                s = _scores(qq, kk[cols], scale, t, cols, causal)  # [L, nc]
                p = np.exp(s - lrow[:, None])
                dv[b, c0:c0 + len(cols), gi] += p.T @ dd_o
                ds = _dsoftmax(p, dd_o @ vv[cols].T, dsum)
                dk[b, c0:c0 + len(cols), gi] += scale * (ds.T @ qq)
    return dq, dk, dv, o, lse


def _dsoftmax(p, dp, dd):
    """Gradient through the row softmax: dS = P * (dP - D)."""
    return p * (dp - dd[:, None])


def merge_lse(o_a, lse_a, o_b, lse_b):
    """Combine two partial attention results over disjoint key sets.

    With lse = log sum exp over each set, the union has
    lse = M + log(exp(lse_a - M) + exp(lse_b - M)), M = max(lse_a, lse_b), and
    O = exp(lse_a - lse) O_a + exp(lse_b - lse) O_b. A partial with lse = -inf
    (no visible key) has weight 0; two such give lse = -inf and O = 0.
    This is the online-softmax correction of the blog's blockwise listing
    (section "ブロック単位の分割戦略") written for normalised partials.
    """
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    m = np.maximum(lse_a, lse_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.exp(lse_a - m_safe)
    wb = np.exp(lse_b - m_safe)
    tot = wa + wb
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = m_safe + np.log(tot)
        o = (wa[..., None] * o_a + wb[..., None] * o_b) / tot[..., None]
    o = np.where((tot == 0)[..., None], 0.0, o)
    return o, lse


def blockwise_ring_fwd(q, k, v, P, rank, layout, causal, scale=None):
    """The pages' online-softmax loop for one device, in ring order, float64.

    Used only to check the method's identity (blockwise == full softmax) in
    the oracle's own tests. q, k, v are original-order [B, L, H, d]; the
    device's query block and each KV block j = (rank - k) mod P are gathered
    through the layout's index map. Per step (blog, "ブロック単位の分割戦略"
    and "リングトポロジーと KV の循環"): new_max = max(max, rowmax S);
    correction = exp(max - new_max); sum = sum*correction + rowsum exp(S -
    new_max); acc = acc*correction + exp(S - new_max) V. A row with no visible
    key in a block keeps its state (the -inf max is rescaled as 0). Returns
    (O, lse) of the block in its local row order.
    """
    from .ring import layout_perm, ring_schedule

    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, L, H, d = q.shape
    Bb = L // P
    _kv_group(H, k.shape[2])
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    perm = layout_perm(L, P, layout)
    rows = perm[rank * Bb:(rank + 1) * Bb]
    o = np.zeros((B, Bb, H, d))
    lse = np.zeros((B, Bb, H))
    for b in range(B):
        for h in range(H):
            hk = _kv_head(h, H, k.shape[2])
            qi = q[b, rows, h, :]
            mx = np.full(Bb, NEG_INF)
            sm = np.zeros(Bb)
            acc = np.zeros((Bb, d))
            for j in ring_schedule(P, rank):
                cols = perm[j * Bb:(j + 1) * Bb]
                s = _scores(qi, k[b, cols, hk, :], scale, rows, cols, causal)
                new_max = np.maximum(mx, s.max(axis=1))
                safe = np.where(np.isfinite(new_max), new_max, 0.0)
                corr = np.exp(mx - safe)
                e = np.exp(s - safe[:, None])
                sm = sm * corr + e.sum(axis=1)
                acc = acc * corr[:, None] + e @ v[b, cols, hk, :]
                mx = new_max
            o[b, :, h] = acc / sm[:, None]
            lse[b, :, h] = mx + np.log(sm)
    return o, lse
