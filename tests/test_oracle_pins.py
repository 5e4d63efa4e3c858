"""Pins of the float64 CPU oracle against facts that do not come from it.

Each test checks the oracle against something independent: scalar brute
force, closed forms, a library routine (torch's CPU float64 attention and its
autograd), finite differences, mathematical identities, the method's own
invariant (blockwise online softmax in ring order equals the full softmax),
permutation equivariance of the striped layout, and values the pages print.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (attention_bwd, attention_fwd, blockwise_ring_fwd, layout_perm, merge_lse)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- brute force

def brute_attention(q, k, v, causal, scale):
    """Scalar loops with math.exp, straight from softmax(scale*QK^T) V."""
    B, L, H, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, L, H))
    for b, h, t in itertools.product(range(B), range(H), range(L)):
        keys = [u for u in range(L) if (u <= t or not causal)]
        sc = [scale * sum(q[b, t, h, e] * k[b, u, h, e] for e in range(d)) for u in keys]
        z = sum(math.exp(s) for s in sc)
        lse[b, t, h] = math.log(z)
        for e in range(d):
            o[b, t, h, e] = sum(math.exp(s) / z * v[b, u, h, e] for s, u in zip(sc, keys))
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_matches_brute_force(causal):
    q, k, v = rnd(1, 2, 7, 2, 3), rnd(2, 2, 7, 2, 3), rnd(3, 2, 7, 2, 3)
    scale = 0.7
    o, lse = attention_fwd(q, k, v, causal, scale=scale, row_chunk=3)
    ob, lb = brute_attention(q, k, v, causal, scale)
    assert np.max(np.abs(o - ob)) < 1e-13
    assert np.max(np.abs(lse - lb)) < 1e-13


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = rnd(4, 1, 5, 1, 4), rnd(5, 1, 5, 1, 4), rnd(6, 1, 5, 1, 4)
    o1, l1 = attention_fwd(q, k, v, True)
    o2, l2 = brute_attention(q, k, v, True, 0.5)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(causal):
    q, k = rnd(7, 1, 33, 2, 8), rnd(8, 1, 33, 2, 8)
    c = rnd(9, 2, 8)
    v = np.broadcast_to(c[None, None], (1, 33, 2, 8)).copy()
    o, _ = attention_fwd(q, k, v, causal, row_chunk=10)
    assert np.max(np.abs(o - v)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_visible_values(causal):
    L = 40
    q, v = rnd(10, 1, L, 3, 4), rnd(11, 1, L, 3, 4)
    k = np.zeros_like(q)
    o, lse = attention_fwd(q, k, v, causal, row_chunk=16)
    if causal:
        cnt = np.arange(1, L + 1, dtype=np.float64)
        exp_o = np.cumsum(v, axis=1) / cnt[None, :, None, None]
    else:
        cnt = np.full(L, float(L))
        exp_o = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    assert np.max(np.abs(o - exp_o)) < 1e-13
    assert np.max(np.abs(lse - np.log(cnt)[None, :, None])) < 1e-13


def test_single_token():
    q, k, v = rnd(12, 1, 1, 2, 6), rnd(13, 1, 1, 2, 6), rnd(14, 1, 1, 2, 6)
    for causal in (False, True):
        o, lse = attention_fwd(q, k, v, causal)
        assert np.max(np.abs(o - v)) == 0.0
        expect = (q * k).sum(-1) / math.sqrt(6)
        assert np.max(np.abs(lse - expect)) < 1e-15


def test_dominant_key_selects_its_value():
    """One key aligned with a large query picks out its own value row."""
    L, d = 9, 4
    q = np.zeros((1, L, 1, d))
    k = np.zeros((1, L, 1, d))
    v = rnd(15, 1, L, 1, d)
    q[0, :, 0, 0] = 60.0
    k[0, 3, 0, 0] = 60.0  # score 1800 vs 0 for every other key
    o, _ = attention_fwd(q, k, v, False, scale=0.5)
    assert np.max(np.abs(o[0, :, 0] - v[0, 3, 0])) < 1e-12
    o, _ = attention_fwd(q, k, v, True, scale=0.5)
    # rows before token 3 cannot see it: plain mean of their visible values
    for t in range(3):
        assert np.max(np.abs(o[0, t, 0] - v[0, :t + 1, 0].mean(0))) < 1e-13
    assert np.max(np.abs(o[0, 3:, 0] - v[0, 3, 0])) < 1e-12


def test_probabilities_sum_to_one_and_are_causal():
    """O = P V with V = identity exposes P: rows sum to 1, future keys get 0."""
    L = 12
    q = rnd(16, 1, L, 1, L)
    k = rnd(17, 1, L, 1, L)
    v = np.eye(L)[None, :, None, :]
    o, _ = attention_fwd(q, k, v, True, row_chunk=5)
    p = o[0, :, 0, :]
    assert np.max(np.abs(p.sum(1) - 1.0)) < 1e-14
    assert np.all(p[np.triu_indices(L, 1)] == 0.0)
    assert np.all(p[np.tril_indices(L)] > 0.0)


# ---------------------------------------------------------------- library routine

torch = pytest.importorskip("torch")


def _torch_sdpa(q, k, v, causal):
    t = lambda x: torch.tensor(x).permute(0, 2, 1, 3).contiguous()  # [B,H,L,d]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    return out.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_matches_torch_cpu_f64(causal):
    q, k, v = rnd(20, 2, 70, 3, 16), rnd(21, 2, 70, 3, 16), rnd(22, 2, 70, 3, 16)
    o, _ = attention_fwd(q, k, v, causal, row_chunk=32)
    assert np.max(np.abs(o - _torch_sdpa(q, k, v, causal))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_matches_torch_autograd_f64(causal):
    q, k, v, do = (rnd(s, 1, 50, 2, 8) for s in (23, 24, 25, 26))
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    g = lambda x: x.grad.permute(0, 2, 1, 3).numpy()
    dq, dk, dv, o, _ = attention_bwd(q, k, v, do, causal, row_chunk=16)
    assert np.max(np.abs(dq - g(tq))) < 1e-12
    assert np.max(np.abs(dk - g(tk))) < 1e-12
    assert np.max(np.abs(dv - g(tv))) < 1e-12


# ---------------------------------------------------------------- backward: calculus and identities

@pytest.mark.parametrize("causal,scale", [(False, None), (True, None), (True, 0.07), (False, 1.3)])
def test_bwd_matches_finite_differences(causal, scale):
    """The gradient of <dO, O> by central differences, at the default scale
    and at explicit ones (a caller's own scale enters dQ and dK once more)."""
    L, d = 6, 3
    q, k, v, do = (rnd(s, 1, L, 1, d) for s in (30, 31, 32, 33))
    dq, dk, dv, _, _ = attention_bwd(q, k, v, do, causal, scale=scale)

    def f(qq, kk, vv):
        return float((attention_fwd(qq, kk, vv, causal, scale=scale)[0] * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = f(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = f(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        rel = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(g)))
        assert rel < 1e-6, (name, rel)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_column_identities(causal):
    """sum_t dK[t] = 0 (each dS row sums to zero) and sum_t dV[t] = sum_t dO[t]
    (each probability row sums to one)."""
    q, k, v, do = (rnd(s, 2, 37, 2, 5) for s in (40, 41, 42, 43))
    dq, dk, dv, _, _ = attention_bwd(q, k, v, do, causal, row_chunk=8)
    assert np.max(np.abs(dk.sum(axis=1))) < 1e-12
    assert np.max(np.abs(dv.sum(axis=1) - do.sum(axis=1))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sampled_equals_full(causal):
    """Row/column-sampled gradients equal the corresponding rows of the full
    backward (which is pinned to autograd and finite differences above)."""
    q, k, v, do = (rnd(s, 2, 41, 3, 5) for s in (48, 49, 80, 81))
    full = attention_bwd(q, k, v, do, causal, heads=[2, 0], row_chunk=9)
    qr, kr = np.array([0, 7, 40, 13]), np.array([40, 0, 22, 5, 6])
    dq, dk, dv, _, _ = oracle.attention_bwd_sampled(q, k, v, do, causal, qr, kr, heads=[2, 0], row_chunk=3)
    assert np.max(np.abs(dq - full[0][:, qr])) < 1e-13
    assert np.max(np.abs(dk - full[1][:, kr])) < 1e-13
    assert np.max(np.abs(dv - full[2][:, kr])) < 1e-13


def test_bwd_head_subset_equals_full():
    q, k, v, do = (rnd(s, 1, 20, 4, 4) for s in (44, 45, 46, 47))
    full = attention_bwd(q, k, v, do, True)
    sub = attention_bwd(q, k, v, do, True, heads=[3, 1])
    for a, b in zip(full[:3], sub[:3]):
        assert np.array_equal(a[:, :, [3, 1]], b)


# ---------------------------------------------------------------- grouped-query attention
# K/V with Hk heads shared by H = G * Hk query heads (query head h reads K/V
# head h // G). torch's enable_gqa attention repeats each K/V head G times
# consecutively, which is the same assignment.

def _torch_sdpa_gqa(q, k, v, causal, do=None):
    t = lambda x: torch.tensor(x).permute(0, 2, 1, 3).contiguous().requires_grad_(do is not None)
    tq, tk, tv = t(q), t(k), t(v)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, enable_gqa=True)
    back = lambda x: x.permute(0, 2, 1, 3).detach().numpy()
    if do is None:
        return back(out)
    out.backward(torch.tensor(do).permute(0, 2, 1, 3))
    return back(out), back(tq.grad), back(tk.grad), back(tv.grad)


@pytest.mark.parametrize("hk", [1, 2, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_fwd_matches_torch_cpu_f64(causal, hk):
    q = rnd(300, 2, 45, 6, 8)
    k, v = rnd(301, 2, 45, hk, 8), rnd(302, 2, 45, hk, 8)
    o, _ = attention_fwd(q, k, v, causal, row_chunk=16)
    assert np.max(np.abs(o - _torch_sdpa_gqa(q, k, v, causal))) < 1e-12


@pytest.mark.parametrize("hk", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_bwd_matches_torch_autograd_f64(causal, hk):
    q, do = rnd(303, 1, 33, 4, 8), rnd(304, 1, 33, 4, 8)
    k, v = rnd(305, 1, 33, hk, 8), rnd(306, 1, 33, hk, 8)
    _, tdq, tdk, tdv = _torch_sdpa_gqa(q, k, v, causal, do)
    dq, dk, dv, _, _ = attention_bwd(q, k, v, do, causal, row_chunk=10)
    assert dk.shape == k.shape and dv.shape == v.shape
    assert np.max(np.abs(dq - tdq)) < 1e-12
    assert np.max(np.abs(dk - tdk)) < 1e-12
    assert np.max(np.abs(dv - tdv)) < 1e-12


def test_gqa_bwd_matches_finite_differences():
    """The gradient of a shared K/V head collects every query head that reads it."""
    L, d = 5, 2
    q, do = rnd(310, 1, L, 4, d), rnd(311, 1, L, 4, d)
    k, v = rnd(312, 1, L, 2, d), rnd(313, 1, L, 2, d)
    dq, dk, dv, _, _ = attention_bwd(q, k, v, do, True)
    f = lambda qq, kk, vv: float((attention_fwd(qq, kk, vv, True)[0] * do).sum())
    h = 1e-6
    for name, x, g in (("k", k, dk), ("v", v, dv), ("q", q, dq)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            fp = f(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = f(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - g)) / np.max(np.abs(g)) < 1e-6, name


def test_mqa_zero_keys_give_prefix_means_for_every_head():
    """One K/V head (multi-query) with K = 0: every query head gets the causal
    prefix mean of the single V head, and lse = ln(visible count)."""
    L = 9
    q, v = rnd(320, 1, L, 5, 4), rnd(321, 1, L, 1, 4)
    o, lse = attention_fwd(q, np.zeros((1, L, 1, 4)), v, True)
    means = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(5):
        assert np.max(np.abs(o[0, :, h] - means)) < 1e-14
        assert np.max(np.abs(lse[0, :, h] - np.log(np.arange(1, L + 1)))) < 1e-14


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_gqa_blockwise_ring_equals_full_softmax(layout):
    L, P = 24, 4
    q, k, v = rnd(330, 1, L, 4, 4), rnd(331, 1, L, 2, 4), rnd(332, 1, L, 2, 4)
    of, lf = attention_fwd(q, k, v, True)
    perm = layout_perm(L, P, layout)
    Bb = L // P
    for rank in range(P):
        ob, lb = blockwise_ring_fwd(q, k, v, P, rank, layout, True)
        rows = perm[rank * Bb:(rank + 1) * Bb]
        assert np.max(np.abs(ob - of[:, rows])) < 1e-12
        assert np.max(np.abs(lb - lf[:, rows])) < 1e-12


def test_gqa_sampled_equals_full_and_needs_whole_groups():
    q, do = rnd(340, 1, 30, 6, 4), rnd(341, 1, 30, 6, 4)
    k, v = rnd(342, 1, 30, 2, 4), rnd(343, 1, 30, 2, 4)
    full = attention_bwd(q, k, v, do, True, heads=[3, 4, 5, 0, 1, 2], row_chunk=7)
    qr, kr = np.array([29, 0, 11]), np.array([0, 17, 29, 4])
    dq, dk, dv, _, _ = oracle.attention_bwd_sampled(q, k, v, do, True, qr, kr, heads=[3, 4, 5, 0, 1, 2])
    assert np.max(np.abs(dq - full[0][:, qr])) < 1e-13
    assert np.max(np.abs(dk - full[1][:, kr])) < 1e-13
    assert np.max(np.abs(dv - full[2][:, kr])) < 1e-13
    ref = attention_bwd(q, k, v, do, True)
    assert np.max(np.abs(full[1] - ref[1][:, :, [1, 0]])) < 1e-13  # groups in order of first appearance
    with pytest.raises(ValueError):
        attention_bwd(q, k, v, do, True, heads=[0, 1])
    with pytest.raises(ValueError):
        attention_fwd(q, rnd(344, 1, 30, 4, 4), rnd(345, 1, 30, 4, 4), True)


def test_planted_interleaved_head_map_is_caught(monkeypatch):
    """Reading K/V head h mod Hk instead of h // G fails the library pin."""
    import oracle.attention as oa
    q, k, v = rnd(350, 1, 12, 4, 4), rnd(351, 1, 12, 2, 4), rnd(352, 1, 12, 2, 4)
    ref = _torch_sdpa_gqa(q, k, v, True)
    monkeypatch.setattr(oa, "_kv_head", lambda h, H, Hk: h % Hk)
    o, _ = oa.attention_fwd(q, k, v, True)
    assert np.max(np.abs(o - ref)) > 1e-3


# ---------------------------------------------------------------- the method's invariant

@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_ring_equals_full_softmax(layout, causal):
    """Online softmax over KV blocks in ring order, for every block count
    dividing L and every rank, equals the full softmax."""
    L = 24
    q, k, v = rnd(50, 1, L, 2, 4), rnd(51, 1, L, 2, 4), rnd(52, 1, L, 2, 4)
    o_full, lse_full = attention_fwd(q, k, v, causal)
    for P in [p for p in range(1, L + 1) if L % p == 0 and (layout != "zigzag" or (L // p) % 2 == 0)]:
        perm = layout_perm(L, P, layout)
        Bb = L // P
        for r in range(P):
            o, lse = blockwise_ring_fwd(q, k, v, P, r, layout, causal)
            rows = perm[r * Bb:(r + 1) * Bb]
            assert np.max(np.abs(o - o_full[:, rows])) < 1e-12, (P, r)
            assert np.max(np.abs(lse - lse_full[:, rows])) < 1e-12, (P, r)


def test_striped_permutation_equivariance():
    """Striped causal attention computed on permuted rows with their original
    positions, permuted back, equals contiguous causal attention."""
    L, P = 48, 4
    q, k, v = rnd(53, 2, L, 2, 8), rnd(54, 2, L, 2, 8), rnd(55, 2, L, 2, 8)
    perm = layout_perm(L, P, "striped")
    inv = np.argsort(perm)
    o_s, l_s = attention_fwd(q[:, perm], k[:, perm], v[:, perm], True, q_pos=perm, k_pos=perm, row_chunk=7)
    o_c, l_c = attention_fwd(q, k, v, True)
    assert np.max(np.abs(o_s[:, inv] - o_c)) < 1e-13
    assert np.max(np.abs(l_s[:, inv] - l_c)) < 1e-13


def test_zigzag_permutation_equivariance():
    """Zigzag causal attention on the blocked rows with their original
    positions, permuted back, equals contiguous causal attention."""
    L, P = 48, 4
    q, k, v = rnd(56, 1, L, 2, 8), rnd(57, 1, L, 2, 8), rnd(58, 1, L, 2, 8)
    perm = layout_perm(L, P, "zigzag")
    inv = np.argsort(perm)
    o_z, l_z = attention_fwd(q[:, perm], k[:, perm], v[:, perm], True, q_pos=perm, k_pos=perm, row_chunk=5)
    o_c, l_c = attention_fwd(q, k, v, True)
    assert np.max(np.abs(o_z[:, inv] - o_c)) < 1e-13
    assert np.max(np.abs(l_z[:, inv] - l_c)) < 1e-13


# ---------------------------------------------------------------- LSE merge

@pytest.mark.parametrize("causal", [False, True])
def test_merge_of_disjoint_key_sets_equals_full(causal):
    L = 30
    q, k, v = rnd(60, 1, L, 2, 6), rnd(61, 1, L, 2, 6), rnd(62, 1, L, 2, 6)
    sel = np.random.default_rng(63).random(L) < 0.4
    a, b = np.flatnonzero(sel), np.flatnonzero(~sel)
    oa, la = attention_fwd(q, k[:, a], v[:, a], causal, k_pos=a)
    ob, lb = attention_fwd(q, k[:, b], v[:, b], causal, k_pos=b)
    assert np.isneginf(la).any() or np.isneginf(lb).any() or not causal
    o, lse = merge_lse(oa, la, ob, lb)
    of, lf = attention_fwd(q, k, v, causal)
    assert np.max(np.abs(o - of)) < 1e-13
    assert np.max(np.abs(lse - lf)) < 1e-13


def test_merge_with_empty_partial_is_identity():
    o, l = rnd(64, 5, 3), rnd(65, 5)
    empty_l = np.full(5, -np.inf)
    o2, l2 = merge_lse(o, l, np.zeros((5, 3)), empty_l)
    assert np.array_equal(l2, l) and np.max(np.abs(o2 - o)) < 1e-15
    o3, l3 = merge_lse(np.zeros((5, 3)), empty_l, np.zeros((5, 3)), empty_l)
    assert np.all(np.isneginf(l3)) and np.all(o3 == 0)


# ---------------------------------------------------------------- ring / layout facts the pages state

def test_ring_order_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "ring_order.json")))
    assert oracle.ring_schedule(4, 0) == g["device0_view_P4"]["blocks"]
    assert [oracle.ring_schedule(4, i)[1] for i in range(4)] == g["step1_table_N4"]["received_block_per_device"]
    # every step is a permutation of blocks over devices; every device sees all blocks
    for P in (1, 2, 5, 8, 16):
        sched = [oracle.ring_schedule(P, i) for i in range(P)]
        for kstep in range(P):
            assert sorted(s[kstep] for s in sched) == list(range(P))
        for s in sched:
            assert sorted(s) == list(range(P))


def test_tick_demo_matches_printed_output():
    """The chapter prints the demo's output: each step's compute and hop
    intervals and the totals for c = 3, m = 1 on 4 devices, and the block
    visits of each device under both assignments of 32 rows."""
    g = json.load(open(os.path.join(GOLDEN, "ring_tick_demo.json")))
    p = g["params"]
    for key, overlap in (("non_overlapped", False), ("overlapped", True)):
        sch = oracle.tick_schedule(p["P"], p["c"], p["m"], overlap)
        assert sch["total"] == g[key]["total"]
        got = [[k, sch["compute"][k].tolist(), sch["hop"][k].tolist()] for k in range(p["P"])]
        assert got == g[key]["steps"]
        assert sch["block"].tolist() == oracle.ring_schedule(p["P"], 0)
    P, B = p["P"], p["block_len"]
    N = P * B
    wc = oracle.block_visits([r // B for r in range(N)], P, B)
    ws = oracle.block_visits([r % P for r in range(N)], P, B)
    assert wc == g["work_contiguous"] and ws == g["work_striped"]
    assert f"{max(wc) / min(wc):.2f}" == g["ratio_contiguous"]
    assert f"{max(ws) / min(ws):.2f}" == g["ratio_striped"]
    assert sum(wc) == sum(ws) == g["total_work"]


def test_tick_model_closed_forms():
    """The ring takes P (c + m) ticks serially and P max(c, m) overlapped;
    overlapped, every hop lies inside its step, and when m <= c the hop is
    entirely hidden (each step ends when its compute ends)."""
    for P, c, m in ((1, 5, 2), (8, 3, 7), (5, 4, 4), (3, 2, 9)):
        ser = oracle.tick_schedule(P, c, m, False)
        ovl = oracle.tick_schedule(P, c, m, True)
        assert ser["total"] == P * (c + m) and ovl["total"] == P * max(c, m)
        assert np.all(ser["hop"][:, 0] == ser["compute"][:, 1])  # hop after compute
        assert np.all(ovl["hop"][:, 0] == ovl["compute"][:, 0])  # hop alongside
        if m <= c:
            assert ovl["compute"][-1, 1] == ovl["total"]


def test_layout_perm_is_the_stated_assignment():
    L, P = 32, 4
    for layout in ("contiguous", "striped", "zigzag"):
        perm = layout_perm(L, P, layout)
        assert sorted(perm) == list(range(L))
        Bb = L // P
        h = Bb // 2
        for s in range(P):
            rows = perm[s * Bb:(s + 1) * Bb]
            if layout == "striped":
                assert all(t % P == s for t in rows)  # token t -> device t mod P
            elif layout == "zigzag":
                # two half-blocks, symmetric: chunk s and chunk 2P-1-s of 2P
                assert list(rows) == list(range(s * h, (s + 1) * h)) + list(
                    range((2 * P - 1 - s) * h, (2 * P - s) * h))
            else:
                assert list(rows) == list(range(s * Bb, (s + 1) * Bb))
            assert list(rows) == sorted(rows)  # ascending inside a device


def test_block_relation_matches_brute_force():
    cases = list(itertools.product(("contiguous", "striped"), (1, 2, 3, 5), (1, 4, 7)))
    cases += list(itertools.product(("zigzag",), (1, 2, 3, 5), (2, 4, 6)))
    for layout, P, Bb in cases:
        for i, j in itertools.product(range(P), range(P)):
            kind, c = oracle.block_relation(layout, P, Bb, i, j)
            a = np.arange(Bb)[:, None]
            b = np.arange(Bb)[None, :]
            vis = oracle.token_position(layout, P, Bb, j, b) <= oracle.token_position(layout, P, Bb, i, a)
            if kind == "none":
                assert not vis.any()
            elif kind == "all":
                assert vis.all()
            elif kind == "first_half":
                assert np.array_equal(vis, np.broadcast_to(b < c, vis.shape))
            elif kind == "second_half_rows":
                assert np.array_equal(vis, np.broadcast_to(a >= c, vis.shape))
            else:
                assert np.array_equal(vis, (b - a) <= c)
        # contiguous rule as stated: later block skipped, own block triangular, earlier block full
        if layout == "contiguous" and P > 1:
            assert oracle.block_relation(layout, P, Bb, 0, 1)[0] == "none"
            assert oracle.block_relation(layout, P, Bb, 1, 0)[0] == "all"


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_unmasked_pair_counts(layout):
    for P, Bb in ((1, 5), (4, 8), (3, 7), (16, 16)):
        counts = oracle.unmasked_pairs_per_rank(layout, P, Bb)
        L = P * Bb
        assert sum(counts) == L * (L + 1) // 2
        for r in range(P):
            if layout == "contiguous":
                assert counts[r] == Bb * Bb * r + Bb * (Bb + 1) // 2
            else:
                assert counts[r] == (r + 1) * Bb + P * Bb * (Bb - 1) // 2
        # brute force on the smallest cases
        if L <= 64:
            perm = layout_perm(L, P, layout)
            for r in range(P):
                rows = perm[r * Bb:(r + 1) * Bb]
                assert counts[r] == int((perm[None, :] <= rows[:, None]).sum())
    assert oracle.unmasked_pairs_per_rank(layout, 4, 8, causal=False) == [256] * 4


def test_zigzag_pair_counts_are_balanced():
    """Device s's first half-block (chunk s) sees s full chunks and its own
    triangle, its second (chunk 2P-1-s) sees 2P-1-s full chunks and its own
    triangle: (2P-1) h^2 + h(h+1) pairs on every device, h = Bb/2."""
    for P, Bb in ((1, 2), (4, 8), (3, 6), (16, 16), (5, 10)):
        h = Bb // 2
        counts = oracle.unmasked_pairs_per_rank("zigzag", P, Bb)
        assert counts == [(2 * P - 1) * h * h + h * (h + 1)] * P
        L = P * Bb
        assert sum(counts) == L * (L + 1) // 2
        if L <= 64:
            perm = layout_perm(L, P, "zigzag")
            for r in range(P):
                rows = perm[r * Bb:(r + 1) * Bb]
                assert counts[r] == int((perm[None, :] <= rows[:, None]).sum())


# ---------------------------------------------------------------- the pins have teeth

def _mut_strict_mask(qc, kk, scale, tq, tk, causal):
    s = scale * (qc @ kk.T)
    return np.where(tk[None, :] < tq[:, None], s, -np.inf) if causal else s


def _mut_no_scale(qc, kk, scale, tq, tk, causal):
    s = qc @ kk.T
    return np.where(tk[None, :] <= tq[:, None], s, -np.inf) if causal else s


def _mut_reversed_mask(qc, kk, scale, tq, tk, causal):
    s = scale * (qc @ kk.T)
    return np.where(tk[None, :] >= tq[:, None], s, -np.inf) if causal else s


@pytest.mark.parametrize("mutant", [_mut_strict_mask, _mut_no_scale, _mut_reversed_mask])
def test_planted_score_mistakes_are_caught(monkeypatch, mutant):
    """A plausible mistake planted in the oracle's score step fails a pin."""
    import oracle.attention as oa
    q, k, v = rnd(70, 1, 6, 1, 3), rnd(71, 1, 6, 1, 3), rnd(72, 1, 6, 1, 3)
    ob, lb = brute_attention(q, k, v, True, 1 / math.sqrt(3))
    monkeypatch.setattr(oa, "_scores", mutant)
    with np.errstate(all="ignore"):
        o, lse = oa.attention_fwd(q, k, v, True)
    err = np.nanmax(np.abs(o - ob)) if np.isfinite(o).any() else np.inf
    assert not (err < 1e-6 and np.nanmax(np.abs(lse - lb)) < 1e-6)


def test_planted_backward_sign_mistake_is_caught(monkeypatch):
    """Flipping D's sign in dS = P (dP - D) breaks the dK column identity and
    the finite-difference check."""
    import oracle.attention as oa
    q, k, v, do = (rnd(s, 1, 6, 1, 3) for s in (73, 74, 75, 76))
    monkeypatch.setattr(oa, "_dsoftmax", lambda p, dp, dd: p * (dp + dd[:, None]))
    dq, dk, dv, o, lse = oa.attention_bwd(q, k, v, do, True)
    assert np.max(np.abs(dk.sum(axis=1))) > 1e-6
    # finite difference on one entry of q
    h = 1e-6
    qp, qm = q.copy(), q.copy()
    qp[0, 4, 0, 1] += h
    qm[0, 4, 0, 1] -= h
    f = lambda qq: float((oa.attention_fwd(qq, k, v, True)[0] * do).sum())
    assert abs((f(qp) - f(qm)) / (2 * h) - dq[0, 4, 0, 1]) > 1e-6
