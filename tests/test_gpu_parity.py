"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases compare every element; they span several tiles, ragged tails
(block lengths that are not tile multiples), all three layouts, causal and not,
bf16 and fp32, head_dim 64 and 128, single-rank (double-buffered receive)
and rank-range launches, grouped-query and multi-query K/V heads, and
degenerate shapes (one block, one token per block). Bars: max |GPU - oracle| <= 2e-2 for bf16 inputs (fp32 accumulation)
and <= 1e-4 for fp32 inputs, on O, lse, dQ, dK and dV; data movement
(layout gathers, pre-permuted vs strided inputs) must be bit-exact.
"""
import numpy as np
import pytest

import exact_blockwise_attention_amd as ra
import oracle
from gpu_cases import (TOL, Case, assert_close, assert_output_close, lse_to_original, log, payloads,
                       rank_positions, to_device, to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.library()  # the HIP library must load; there is no fallback


def run_fwd(case, dev, rank_range=None, copy=False, split=True, scale=None):
    stream = torch.cuda.Stream() if copy else None
    o, lse = ra.attention_forward(dev["q"], dev["k"], dev["v"], case.P, case.layout, case.causal, scale=scale,
                                  rank_range=rank_range, copy_stream=stream, split=split)
    torch.cuda.synchronize()
    return o, lse


def check_fwd(case, o, lse, ref_o, ref_lse, ranks):
    pos, lse_vals = lse_to_original(case, lse, ranks)
    tol = TOL[case.dtype]
    assert_output_close("O", to_f64(o)[:, pos], ref_o[:, pos], case.dtype, case)
    assert_close("lse", lse_vals, ref_lse[:, pos], tol, case)


SMALL_FWD = [
    Case(101, 1, 2, 1024, 128, 4, False, "contiguous", "bf16"),
    Case(102, 2, 2, 800, 128, 4, True, "contiguous", "bf16"),
    Case(103, 2, 2, 800, 128, 4, True, "striped", "bf16"),
    Case(104, 1, 3, 408, 128, 3, True, "striped", "bf16"),
    Case(105, 1, 2, 650, 64, 5, True, "striped", "bf16"),
    Case(106, 2, 1, 128, 64, 2, True, "contiguous", "bf16"),
    Case(107, 1, 1, 1024, 64, 4, False, "contiguous", "f32"),
    Case(108, 1, 2, 400, 64, 4, True, "striped", "f32"),
    Case(109, 1, 2, 210, 128, 3, True, "contiguous", "f32"),
    Case(110, 1, 2, 300, 128, 1, True, "contiguous", "bf16"),   # one block
    Case(111, 1, 2, 8, 128, 8, True, "striped", "bf16"),        # one token per block
    Case(112, 1, 2, 8, 64, 8, True, "contiguous", "f32"),
    Case(113, 1, 1, 4096, 128, 2, True, "striped", "bf16"),     # many tiles per block
    # zigzag: half-blocks of 100 rows (tiles straddle the halves), 128 rows,
    # fp32, one token per half-block, many tiles per block
    Case(114, 1, 2, 800, 128, 4, True, "zigzag", "bf16"),
    Case(115, 1, 2, 1024, 64, 4, True, "zigzag", "bf16"),
    Case(116, 1, 2, 400, 64, 4, True, "zigzag", "f32"),
    Case(117, 1, 2, 16, 128, 8, True, "zigzag", "bf16"),
    Case(118, 1, 1, 4096, 128, 2, True, "zigzag", "bf16"),
    Case(119, 1, 2, 600, 128, 3, False, "zigzag", "bf16"),
    # grouped-query (Hk K/V heads shared by H query heads) and multi-query
    Case(161, 1, 4, 800, 128, 4, True, "striped", "bf16", Hk=2),
    Case(162, 1, 6, 520, 64, 4, True, "contiguous", "bf16", Hk=1),
    Case(163, 1, 4, 800, 128, 4, True, "zigzag", "bf16", Hk=1),
    Case(164, 1, 4, 400, 64, 4, True, "striped", "f32", Hk=2),
    Case(165, 2, 6, 1024, 128, 2, False, "contiguous", "bf16", Hk=3),
    Case(166, 1, 8, 2048, 128, 2, True, "striped", "bf16", Hk=2),
    # work orders with partial runs: 9 (head, rank) groups (runs of 4 groups
    # end short) and 6 query tiles per block (the last run of 4 tiles is cut)
    Case(167, 1, 3, 4140, 128, 3, True, "striped", "bf16"),
    Case(168, 1, 3, 4140, 128, 3, True, "zigzag", "bf16"),
]


@pytest.mark.parametrize("case", SMALL_FWD, ids=str)
def test_forward_small(case):
    log(f"forward {case}")
    p = payloads(case)
    dev = {n: to_device(x) for n, x in p.items()}
    ref_o, ref_lse = oracle.attention_fwd(*(syn_f64(p[n]) for n in "qkv"), case.causal)
    o, lse = run_fwd(case, dev)
    check_fwd(case, o, lse, ref_o, ref_lse, range(case.P))


def syn_f64(x):
    from exact_blockwise_attention_amd import synthetic as syn
    return syn.to_f64(x)


STEP_CASES = [
    Case(121, 1, 2, 800, 128, 4, True, "striped", "bf16"),
    Case(122, 1, 2, 800, 128, 4, True, "contiguous", "bf16"),
    Case(123, 1, 2, 520, 64, 4, False, "contiguous", "bf16"),
    Case(124, 1, 1, 400, 64, 4, True, "striped", "f32"),
    Case(125, 1, 2, 800, 128, 4, True, "zigzag", "bf16"),
    Case(126, 1, 4, 800, 128, 4, True, "striped", "bf16", Hk=2),
    Case(127, 1, 2, 400, 64, 4, True, "contiguous", "f32", Hk=1),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=str)
def test_forward_single_rank_with_receive_stream(case):
    """One device's share: every ring step's KV block is gathered into a
    double buffer on a second stream; the state is merged between steps."""
    p = payloads(case)
    dev = {n: to_device(x) for n, x in p.items()}
    ref_o, ref_lse = oracle.attention_fwd(*(syn_f64(p[n]) for n in "qkv"), case.causal)
    for r in range(case.P):
        log(f"single rank {r} with receive stream: {case}")
        o, lse = run_fwd(case, dev, rank_range=(r, r + 1), copy=True)
        check_fwd(case, o, lse, ref_o, ref_lse, [r])
        o2, lse2 = run_fwd(case, dev, rank_range=(r, r + 1), copy=False)
        check_fwd(case, o2, lse2, ref_o, ref_lse, [r])
    log(f"rank range [1, 3): {case}")
    o, lse = run_fwd(case, dev, rank_range=(1, 3))
    check_fwd(case, o, lse, ref_o, ref_lse, [1, 2])


def test_forward_is_deterministic_and_grid_independent():
    """Same inputs give bitwise-equal outputs, whether a rank is computed
    alone or with the whole ring in one launch."""
    case = Case(131, 1, 2, 1024, 128, 4, True, "striped", "bf16")
    log(f"determinism {case}")
    dev = {n: to_device(x) for n, x in payloads(case).items()}
    o1, l1 = run_fwd(case, dev)
    o2, l2 = run_fwd(case, dev)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    o3, l3 = run_fwd(case, dev, rank_range=(2, 3), split=False)
    pos = rank_positions(case, [2])[0]
    assert torch.equal(o1[:, pos].view(torch.int16), o3[:, pos].view(torch.int16))
    assert torch.equal(l1[2], l3[0])


SPLIT_CASES = [
    # one rank's share with a small query block: its ring steps run as
    # parallel runs merged by log-sum-exp. Runs of 1, 2 and 3 ring steps,
    # ragged and one-tile blocks, every layout, grouped-query heads
    Case(171, 1, 2, 1024, 128, 8, True, "striped", "bf16"),
    Case(172, 1, 2, 1040, 128, 8, True, "contiguous", "bf16"),
    Case(173, 1, 4, 1200, 128, 6, True, "zigzag", "bf16", Hk=2),
    Case(174, 2, 3, 1500, 64, 5, False, "contiguous", "bf16"),
    Case(175, 1, 8, 16384, 128, 64, False, "contiguous", "bf16"),   # 256-row blocks, 64 steps
    Case(176, 1, 8, 16384, 128, 256, True, "striped", "bf16", Hk=1),  # 64-row blocks, 256 steps
    # query blocks of at most 64 rows: ragged blocks, d = 64, one-token
    # blocks, grouped-query heads, two batches, every layout
    Case(271, 1, 4, 800, 64, 16, True, "striped", "bf16"),              # 50-row blocks
    Case(272, 2, 3, 960, 128, 24, False, "contiguous", "bf16"),         # 40-row blocks
    Case(273, 1, 4, 1024, 128, 16, True, "zigzag", "bf16", Hk=2),       # 64-row blocks
    Case(274, 1, 2, 64, 128, 64, True, "contiguous", "bf16"),           # 1-row blocks
    Case(275, 1, 8, 2048, 64, 32, True, "contiguous", "bf16", Hk=4),    # 64-row blocks, d = 64
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=str)
def test_forward_single_rank_split_runs(case):
    """A single rank's share, split into runs of ring steps and merged,
    against the oracle and against the same share in one unsplit launch."""
    pb = ra.make_problem(case.B, case.H, case.d, case.P, case.Bb, case.layout, case.causal, 1, None,
                         kv_heads=case.kv_heads)
    assert ra.workspace_bytes(pb, 0, 1, False, False) > 0, "the share should be split"
    p = payloads(case)
    dev = {n: to_device(x) for n, x in p.items()}
    q64, k64, v64 = (syn_f64(p[n]) for n in "qkv")
    for r in sorted({0, 1, case.P // 2, case.P - 1}):
        log(f"split single rank {r}: {case}")
        # the oracle on this rank's query rows, at their token positions
        pr = rank_positions(case, [r])[0]
        ref_o, ref_lse = oracle.attention_fwd(q64[:, pr], k64, v64, case.causal, q_pos=pr)
        outs = []
        for split in (True, False):
            o, lse = run_fwd(case, dev, rank_range=(r, r + 1), split=split)
            _, lv = lse_to_original(case, lse, [r])
            assert_output_close("O", to_f64(o)[:, pr], ref_o, case.dtype, case)
            assert_close("lse", lv, ref_lse, TOL[case.dtype], case)
            outs.append((o[:, pr].float(), lse))
        # the two launches round the bf16 probabilities against different
        # running maxima, so they agree to the same bar, not bitwise
        assert float((outs[0][0] - outs[1][0]).abs().max()) <= TOL[case.dtype]
        assert float((outs[0][1] - outs[1][1]).abs().max()) <= TOL[case.dtype]


def test_layout_copy_is_bit_exact():
    case = Case(132, 2, 3, 96, 64, 4, True, "striped", "bf16")
    log(f"layout copy {case}")
    for layout in ("striped", "contiguous", "zigzag"):
        p = payloads(case, ("q",))["q"]
        x = to_device(p)
        blk = ra.layout_copy(x, case.P, layout)
        torch.cuda.synchronize()
        perm = oracle.layout_perm(case.L, case.P, layout)
        expect = p[:, perm].reshape(case.B, case.P, case.Bb, case.H, case.d).transpose(1, 0, 2, 3, 4)
        got = blk.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, expect)
        back = ra.layout_copy(blk, case.P, layout, inverse=True)
        torch.cuda.synchronize()
        assert np.array_equal(back.view(torch.int16).cpu().numpy().view(np.uint16), p)


def test_prepermuted_input_gives_bitwise_equal_output():
    """Striped attention on blocked (pre-permuted) tensors equals, bit for
    bit, striped attention on original-order tensors described by strides."""
    case = Case(133, 1, 2, 1000, 128, 4, True, "striped", "bf16")
    log(f"pre-permuted vs strided {case}")
    dev = {n: to_device(x) for n, x in payloads(case).items()}
    o, lse = run_fwd(case, dev)
    blk = {n: ra.layout_copy(t, case.P, "striped") for n, t in dev.items()}
    o_blk = torch.empty_like(blk["q"])
    lse_blk = torch.empty_like(lse)
    pb = ra.make_problem(case.B, case.H, case.d, case.P, case.Bb, "striped", True, ra.BF16)
    ra.forward_raw(pb, 0, case.P, ra.seq_blocked(blk["q"]), ra.seq_blocked(blk["k"]), ra.seq_blocked(blk["v"]),
                   ra.seq_blocked(o_blk), lse_blk.data_ptr(), None, 0, ra._stream_handle(None), None)
    o_back = ra.layout_copy(o_blk, case.P, "striped", inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_back.view(torch.int16), o.view(torch.int16))
    assert torch.equal(lse_blk, lse)


def test_merge_lse_kernel():
    rng = np.random.default_rng(134)
    rows, d = 1000, 128
    oa, ob = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
    la, lb = rng.standard_normal(rows) * 5, rng.standard_normal(rows) * 5
    la[::7] = -np.inf
    lb[::11] = -np.inf
    ref_o, ref_l = oracle.merge_lse(oa, la, ob, lb)
    t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")  # noqa: E731
    log("merge_lse rows=1000 d=128")
    o, l = ra.merge_lse(t(oa), t(la), t(ob), t(lb))
    torch.cuda.synchronize()
    assert_close("merge O", o.cpu().numpy(), ref_o, 1e-5)
    lg = l.cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert_close("merge lse", lg[fin], ref_l[fin], 1e-5)
    # in place, odd head_dim (scalar path)
    oa3, ob3 = t(oa[:, :37]).contiguous(), t(ob[:, :37]).contiguous()
    la3 = t(la)
    ref_o3, ref_l3 = oracle.merge_lse(oa[:, :37], la, ob[:, :37], lb)
    ra.merge_lse(oa3, la3, ob3, t(lb), out=oa3, lse_out=la3)
    torch.cuda.synchronize()
    assert_close("merge O in place", oa3.cpu().numpy(), ref_o3, 1e-5)
    assert_close("merge lse in place", la3.cpu().numpy()[fin], ref_l3[fin], 1e-5)


SMALL_BWD = [
    Case(141, 1, 2, 800, 128, 4, True, "striped", "bf16"),
    Case(142, 2, 1, 800, 128, 4, True, "contiguous", "bf16"),
    Case(143, 1, 2, 512, 128, 4, False, "contiguous", "bf16"),
    Case(144, 1, 2, 650, 64, 5, True, "striped", "bf16"),
    Case(145, 1, 1, 300, 128, 1, True, "contiguous", "bf16"),
    Case(146, 1, 2, 400, 64, 4, True, "striped", "f32"),
    Case(147, 1, 1, 210, 128, 3, True, "contiguous", "f32"),
    Case(148, 1, 1, 8, 128, 8, True, "striped", "bf16"),
    Case(150, 1, 2, 800, 128, 4, True, "zigzag", "bf16"),
    Case(151, 1, 2, 400, 64, 4, True, "zigzag", "f32"),
    Case(152, 1, 1, 1000, 64, 5, True, "zigzag", "bf16"),
    # grouped-query and multi-query: dK/dV of a K/V head sum over its group
    Case(153, 1, 4, 800, 128, 4, True, "striped", "bf16", Hk=2),
    Case(154, 1, 3, 650, 64, 5, True, "contiguous", "bf16", Hk=1),
    Case(155, 1, 4, 800, 128, 4, True, "zigzag", "bf16", Hk=1),
    Case(156, 1, 4, 400, 64, 4, True, "striped", "f32", Hk=2),
    Case(157, 2, 6, 512, 128, 4, False, "contiguous", "bf16", Hk=3),
    # blocks that end inside a 64-row / 64-key tile without a causal mask:
    # the last tile is the only one the walks treat as partly visible
    Case(158, 1, 2, 600, 128, 4, False, "contiguous", "bf16"),
    Case(159, 1, 2, 344, 64, 4, False, "striped", "bf16", Hk=1),
    Case(160, 1, 4, 1020, 64, 6, True, "zigzag", "bf16", Hk=2),
    # work orders with partial runs: 9 groups, 6 query tiles and 11 key tiles
    # per block; and two query heads per K/V head (turns of unequal heads)
    Case(169, 1, 3, 4140, 128, 3, True, "striped", "bf16"),
    Case(170, 1, 6, 2100, 64, 3, True, "striped", "bf16", Hk=3),
    # rings of more than 32 ranks: the key-side walk holds its (pass, rank)
    # pairs 64 at a time, so these walks cross into a second set of pairs
    Case(171, 1, 2, 4000, 64, 40, True, "striped", "bf16"),
    Case(172, 1, 2, 2520, 128, 36, True, "zigzag", "bf16", Hk=1),
    Case(173, 1, 1, 2112, 128, 33, False, "contiguous", "bf16"),
    Case(174, 1, 1, 2176, 64, 34, True, "contiguous", "bf16"),
]


def run_bwd(case, dev, rank_range=None, scale=None):
    o, lse = run_fwd(case, dev, rank_range=rank_range, scale=scale)
    dq, dk, dv = ra.attention_backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.P, case.layout,
                                       case.causal, scale=scale, rank_range=rank_range)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("case", SMALL_BWD, ids=str)
def test_backward_small(case):
    log(f"backward {case}")
    p = payloads(case, ("q", "k", "v", "do"))
    dev = {n: to_device(x) for n, x in p.items()}
    f = {n: syn_f64(x) for n, x in p.items()}
    dq_r, dk_r, dv_r, _, _ = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], case.causal)
    dq, dk, dv = run_bwd(case, dev)
    tol = TOL[case.dtype]
    assert_output_close("dQ", to_f64(dq), dq_r, case.dtype, case)
    assert_output_close("dK", to_f64(dk), dk_r, case.dtype, case)
    assert_output_close("dV", to_f64(dv), dv_r, case.dtype, case)


MINIMAL_WS = [
    Case(281, 1, 2, 650, 64, 5, True, "striped", "bf16"),
    Case(282, 1, 4, 1024, 128, 4, True, "zigzag", "bf16", Hk=2),
    Case(283, 2, 2, 768, 128, 3, False, "contiguous", "bf16"),
    Case(284, 1, 2, 800, 128, 4, True, "striped", "bf16", Hk=1),
]


@pytest.mark.parametrize("case", MINIMAL_WS, ids=str)
def test_backward_minimal_workspace(case):
    """A caller's workspace of workspace_bytes(..., 2) bytes holds D and the
    lse only, so the library takes the path that stores no dS and recomputes
    S and dP for dQ. Same bar against the oracle as the default path."""
    log(f"backward, minimal workspace {case}")
    p = payloads(case, ("q", "k", "v", "do"))
    dev = {n: to_device(x) for n, x in p.items()}
    f = {n: syn_f64(x) for n, x in p.items()}
    dq_r, dk_r, dv_r, _, _ = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], case.causal)
    o, lse = run_fwd(case, dev)
    Hk = dev["k"].shape[2]
    pb = ra.make_problem(case.B, case.H, case.d, case.P, case.L // case.P, case.layout, case.causal,
                         ra.BF16, None, kv_heads=Hk)
    small = ra.workspace_bytes(pb, 0, case.P, False, 2)
    assert 0 < small < ra.workspace_bytes(pb, 0, case.P, False, True)
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    dq, dk, dv = ra.attention_backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.P, case.layout,
                                       case.causal, workspace=ws)
    torch.cuda.synchronize()
    assert_output_close("dQ", to_f64(dq), dq_r, case.dtype, case)
    assert_output_close("dK", to_f64(dk), dk_r, case.dtype, case)
    assert_output_close("dV", to_f64(dv), dv_r, case.dtype, case)
    # one byte short of the minimum is refused before anything is launched
    with pytest.raises(ra.RaError):
        ra.attention_backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.P, case.layout, case.causal,
                              workspace=torch.empty(small - 1, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("layout,hk", [("striped", 0), ("zigzag", 0), ("striped", 1)])
def test_backward_rank_range(layout, hk):
    """Ranks [1, 3): dQ of their rows, and dK/dV holding only their queries'
    contributions (the oracle's gradient with dO zero outside those rows)."""
    case = Case(149, 1, 2, 800, 128, 4, True, layout, "bf16", Hk=hk)
    log(f"backward rank range [1,3) {case}")
    p = payloads(case, ("q", "k", "v", "do"))
    dev = {n: to_device(x) for n, x in p.items()}
    f = {n: syn_f64(x) for n, x in p.items()}
    pos = rank_positions(case, [1, 2]).reshape(-1)
    do_masked = np.zeros_like(f["do"])
    do_masked[:, pos] = f["do"][:, pos]
    dq_r, dk_r, dv_r, _, _ = oracle.attention_bwd(f["q"], f["k"], f["v"], do_masked, case.causal)
    dq, dk, dv = run_bwd(case, dev, rank_range=(1, 3))
    tol = TOL[case.dtype]
    assert_output_close("dQ", to_f64(dq)[:, pos], dq_r[:, pos], case.dtype, case)
    assert_output_close("dK", to_f64(dk), dk_r, case.dtype, case)
    assert_output_close("dV", to_f64(dv), dv_r, case.dtype, case)


SCALE_CASES = [
    # a caller's own scale (not 1/sqrt(d)): every kernel folds it into its
    # exponent and the backward applies it again to dQ and dK. Gradients grow
    # with the scale (sharper softmax rows), and so does the bf16 operands'
    # rounding error, in proportion; the scales here (0.79 to 1.47 times the
    # default spread of the scores) keep max |dQ|, |dK| within the range of
    # the default-scale cases (below 4.5), where 2e-2 is the bar
    (Case(181, 1, 2, 800, 128, 4, True, "striped", "bf16"), 0.07),
    (Case(182, 1, 2, 800, 128, 4, True, "zigzag", "bf16"), 0.13),
    (Case(188, 1, 2, 800, 64, 4, True, "striped", "bf16"), 0.17),
    (Case(183, 1, 2, 400, 64, 4, True, "striped", "f32"), 0.2),
    (Case(184, 1, 4, 800, 128, 4, True, "zigzag", "bf16", Hk=2), 0.07),
    (Case(185, 1, 2, 600, 64, 3, False, "contiguous", "bf16"), 0.2),
    (Case(186, 1, 2, 400, 128, 4, True, "zigzag", "f32"), 0.07),
]


@pytest.mark.parametrize("case,scale", SCALE_CASES, ids=lambda x: str(x))
def test_explicit_scale_forward_backward(case, scale):
    log(f"explicit scale {scale}: {case}")
    p = payloads(case, ("q", "k", "v", "do"))
    dev = {n: to_device(x) for n, x in p.items()}
    f = {n: syn_f64(x) for n, x in p.items()}
    dq_r, dk_r, dv_r, o_r, lse_r = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], case.causal, scale=scale)
    o, lse = run_fwd(case, dev, scale=scale)
    check_fwd(case, o, lse, o_r, lse_r, range(case.P))
    dq, dk, dv = run_bwd(case, dev, scale=scale)
    assert_output_close("dQ", to_f64(dq), dq_r, case.dtype, case)
    assert_output_close("dK", to_f64(dk), dk_r, case.dtype, case)
    assert_output_close("dV", to_f64(dv), dv_r, case.dtype, case)
    # one rank's share through the receive stream, and split into runs
    r = case.P - 1
    o1, lse1 = run_fwd(case, dev, rank_range=(r, r + 1), copy=True, scale=scale)
    check_fwd(case, o1, lse1, o_r, lse_r, [r])
    o2, lse2 = run_fwd(case, dev, rank_range=(r, r + 1), split=True, scale=scale)
    check_fwd(case, o2, lse2, o_r, lse_r, [r])


def _copy_mode_buffers(ws, case):
    """The receive buffers at the start of a copy-mode forward workspace:
    K0, V0, K1, V1, each a dense [B][block_len][kv_heads][d] block, each
    starting at a multiple of 256 bytes (include/ra.h, ra_forward)."""
    es = 2 if case.dtype == "bf16" else 4
    blk = case.B * case.Bb * case.kv_heads * case.d * es
    step = (blk + 255) // 256 * 256
    out = []
    for i in range(4):
        b = ws[i * step:i * step + blk]
        out.append(b.view(torch.int16 if es == 2 else torch.int32).reshape(case.B, case.Bb, case.kv_heads, case.d))
    return {"k": (out[0], out[2]), "v": (out[1], out[3])}


@pytest.mark.parametrize("delay", ["none", "copy_stream_late", "inputs_written_late"])
def test_receive_stream_ordering(delay):
    """The receive stand-in's three ordering edges, each under a delay that
    would expose a missing wait ("Ring Attention 論文分析", section on
    limitations and failure cases: a receiver computing on the previous
    round's buffer is silent corruption). The workspace, which holds the
    double buffer, starts as NaN.
      copy_stream_late: the copy stream is held back by a spin, so every step
        must wait for its block's copy (read after write);
      inputs_written_late: K and V start as NaN and receive their values on
        the compute stream after a spin, so the first copy must wait for the
        inputs to be ready on the compute stream;
      write after read: a step's kernel outlasts the copies many times over
        (checked below), so a copy that did not wait for the step that last
        read its buffer would overwrite that buffer while it is read.
    The output must match the oracle, and the last two blocks left in the
    buffers must equal the striped blocks x[:, j::P] bit for bit."""
    case = Case(187, 1, 8, 32768, 128, 4, True, "striped", "bf16")
    P, Bb, r = case.P, case.Bb, case.P - 1
    log(f"receive ordering ({delay}): {case} rank {r}")
    p = payloads(case)
    dev = {n: to_device(x) for n, x in p.items()}
    pb = ra.make_problem(case.B, case.H, case.d, P, Bb, case.layout, True, ra.BF16)
    need = ra.workspace_bytes(pb, r, r + 1, True, False)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN in bf16 and fp32
    copy = torch.cuda.Stream()
    spin = 40_000_000  # clock cycles: about 20 ms
    k_in, v_in = dev["k"], dev["v"]
    if delay == "inputs_written_late":
        k_in = torch.full_like(dev["k"], float("nan"))
        v_in = torch.full_like(dev["v"], float("nan"))
    torch.cuda.synchronize()
    if delay == "copy_stream_late":
        with torch.cuda.stream(copy):
            torch.cuda._sleep(spin)
    if delay == "inputs_written_late":
        torch.cuda._sleep(spin)
        k_in.copy_(dev["k"])
        v_in.copy_(dev["v"])
    o, lse = ra.attention_forward(dev["q"], k_in, v_in, P, case.layout, True, rank_range=(r, r + 1),
                                  copy_stream=copy, workspace=ws)
    torch.cuda.synchronize()
    # the oracle on sampled rows of rank r, heads 0 and H-1
    pos_r = rank_positions(case, [r])[0]
    rows = np.unique(np.concatenate([[0, Bb - 1], np.random.default_rng(187).choice(Bb, 254, replace=False)]))
    heads = [0, case.H - 1]
    f = {n: syn_f64(np.ascontiguousarray(p[n][:, :, heads])) for n in "qkv"}
    ref_o, ref_lse = oracle.attention_fwd(f["q"][:, pos_r[rows]], f["k"], f["v"], True, q_pos=pos_r[rows])
    got_o = to_f64(o[:, torch.as_tensor(pos_r[rows], device="cuda")][:, :, heads])
    got_lse = lse.cpu().numpy()[0][:, heads][:, :, rows].transpose(0, 2, 1)
    assert_output_close("O", got_o, ref_o, case.dtype, case)
    assert_close("lse", got_lse, ref_lse, TOL[case.dtype], case)
    # the buffers hold the blocks of the last two ring steps, bit for bit
    bufs = _copy_mode_buffers(ws, case)
    for step in (P - 2, P - 1):
        j = (r - step) % P
        for n in "kv":
            want = p[n][:, j::P]  # striped block j: tokens j, j + P, ...
            got = bufs[n][step & 1].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want), f"{n} block {j} (step {step}) differs from its source"
    if delay == "none":
        # write after read is exercised: one step's kernel takes many times
        # longer than the copies of a block (K and V)
        t = {}
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        ra.attention_forward(dev["q"], dev["k"], dev["v"], P, case.layout, True, rank_range=(r, r + 1), split=False)
        ev[1].record()
        ra.layout_copy(dev["k"], P, case.layout)
        ra.layout_copy(dev["v"], P, case.layout)
        ev[2].record()
        torch.cuda.synchronize()
        t["step"] = ev[0].elapsed_time(ev[1]) / P
        t["copy"] = ev[1].elapsed_time(ev[2]) / P  # K and V of one block
        log(f"  one step {t['step']:.3f} ms, one block's copies {t['copy']:.3f} ms")
        assert t["step"] > 4 * t["copy"]
