"""The C-ABI library loads on a machine without a GPU, exports every function
include/ra.h declares, and rejects invalid arguments before touching HIP.

None of these calls reaches the GPU: every checked call fails validation,
which the library performs before its first HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

import exact_blockwise_attention_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ra.library_path),
                                reason="libra.so not built (python -m exact_blockwise_attention_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_functions():
    assert declared_functions() == sorted(ra.EXPORTED_FUNCTIONS)


def test_library_exports_every_declared_symbol():
    lib = ra.library()
    out = subprocess.run(["nm", "-D", "--defined-only", ra.library_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ra_[a-z_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings_and_version():
    assert ra.abi_version() == 3
    assert ra.status_string(0) == "ok"
    for code in range(1, 8):
        assert ra.status_string(code) not in ("ok", "unknown status")
    assert ra.status_string(99) == "unknown status"


def problem(**kw):
    base = dict(B=1, H=2, d=64, P=4, Bb=64, layout="striped", causal=True, dtype_code=ra.BF16, kv_heads=0)
    base.update(kw)
    return ra.make_problem(base["B"], base["H"], base["d"], base["P"], base["Bb"], base["layout"],
                           base["causal"], base["dtype_code"], kv_heads=base["kv_heads"])


def fake_seq(ptr=0x10000, s_blk=128, s_batch=1 << 20, s_tok=512, s_head=64):
    return ra.Seq(ptr, s_blk, s_batch, s_tok, s_head)


def fwd_status(pb, rb=0, re_=None, seqs=None, lse=0x20000, ws=None, ws_bytes=0, copy=None):
    re_ = pb.ring_size if re_ is None else re_
    q, k, v, o = seqs or [fake_seq() for _ in range(4)]
    lib = ra.library()
    return lib.ra_forward(ctypes.byref(pb), rb, re_, ra._ref(q), ra._ref(k), ra._ref(v), ra._ref(o),
                          lse, ws, ws_bytes, None, copy)


def test_workspace_sizes():
    pb = problem(d=128, P=8, Bb=4096, H=32)
    assert ra.workspace_bytes(pb, 0, 8, False, False) == 0
    blk = 1 * 4096 * 32 * 128 * 2
    rows = 1 * 32 * 4096
    expect_fwd = 4 * blk + rows * 128 * 4 + rows * 4  # all multiples of 256 here
    assert ra.workspace_bytes(pb, 7, 8, True, False) == expect_fwd
    rows8 = 8 * rows
    assert ra.workspace_bytes(pb, 0, 8, False, 2) == rows8 * 8  # D = rowsum(dO * O) and lse * log2(e)
    # the full backward workspace adds K in operand order and the stored dS tiles
    assert ra.workspace_bytes(pb, 0, 8, False, True) > 30 * rows8 * 8 * 128
    assert ra.workspace_bytes(problem(d=96), 0, 4, False, True) == 0  # invalid problem


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, 2), ("heads", 0, 2), ("ring_size", 0, 2), ("block_len", 0, 2),
    ("layout", 3, 2), ("causal", 3, 2), ("dtype", 7, 2), ("head_dim", 96, 3), ("head_dim", 32, 3),
    ("kv_heads", 3, 2), ("kv_heads", -1, 2),
])
def test_invalid_problem_fields(field, value, code):
    pb = problem()
    setattr(pb, field, value)
    assert fwd_status(pb) == code


def test_split_launch_workspace():
    """One rank whose query tiles (256 rows) number fewer than 256 asks for
    the partial states of its split launch: S = min(P, ceil(256 / tiles))
    runs, each an fp32 O and lse per query row (256-byte aligned parts)."""
    def align(x):
        return (x + 255) // 256 * 256
    pb = problem(d=128, P=256, Bb=64, H=8, causal=False, layout="contiguous")
    rows = 32 * 8 * 64  # 32 runs of the rank's 8 x 64 rows
    assert ra.workspace_bytes(pb, 5, 6, False, False) == align(rows * 128 * 4) + align(rows * 4)
    pb3 = problem(d=64, P=3, Bb=300, H=2)  # 2 query tiles per head: 4 tiles, 3 runs (all P steps)
    rows3 = 3 * 2 * 300
    assert ra.workspace_bytes(pb3, 2, 3, False, False) == align(rows3 * 64 * 4) + align(rows3 * 4)
    assert ra.workspace_bytes(pb, 0, 2, False, False) == 0  # more than one rank: one launch
    assert ra.workspace_bytes(problem(d=128, P=256, Bb=64, H=8, dtype_code=ra.F32), 0, 1, False, False) == 0
    assert ra.workspace_bytes(problem(d=128, P=1, Bb=64, H=8), 0, 1, False, False) == 0
    assert ra.workspace_bytes(problem(d=128, P=8, Bb=4096, H=32), 7, 8, False, False) == 0  # fills the GPU
    # a split-sized workspace must be aligned; checked before anything is launched
    need = ra.workspace_bytes(pb3, 2, 3, False, False)
    assert fwd_status(pb3, 2, 3, ws=0x40010, ws_bytes=need) == 5  # RA_ERR_ALIGN


def test_grouped_query_heads():
    # K/V heads must divide the query heads; the receive buffers of the
    # single-rank forward hold K/V blocks with the K/V head count
    pb = problem(d=128, P=8, Bb=4096, H=32, kv_heads=8)
    blk_kv = 1 * 4096 * 8 * 128 * 2
    rows = 1 * 32 * 4096
    assert ra.workspace_bytes(pb, 7, 8, True, False) == 4 * blk_kv + rows * 128 * 4 + rows * 4
    assert ra.workspace_bytes(pb, 0, 8, False, 2) == 8 * rows * 8  # D and lse2: one row per query head
    assert ra.workspace_bytes(problem(H=32, kv_heads=1), 0, 4, False, True) > 0  # multi-query
    assert ra.workspace_bytes(problem(H=32, kv_heads=12), 0, 4, False, True) == 0
    assert ra.workspace_bytes(problem(H=4, kv_heads=8), 0, 4, False, True) == 0


def test_zigzag_needs_an_even_block_length():
    assert fwd_status(problem(layout="zigzag", Bb=63)) == 2
    # validation only (nothing is launched): a valid problem has a backward
    # workspace, an invalid one reports 0 bytes
    assert ra.workspace_bytes(problem(layout="zigzag", Bb=64), 0, 4, False, True) > 0
    assert ra.workspace_bytes(problem(layout="zigzag", Bb=63), 0, 4, False, True) == 0


def test_forward_token_stride_limit():
    # the bf16 forward addresses a 64-row K/V tile with 32-bit byte offsets
    big = fake_seq(s_tok=(1 << 25) + 8)
    seqs = [fake_seq(), big, fake_seq(), fake_seq()]
    assert fwd_status(problem(), seqs=seqs) == 3
    seqs = [fake_seq(), fake_seq(), big, fake_seq()]
    assert fwd_status(problem(), seqs=seqs) == 3


def test_invalid_scale_nan():
    pb = problem()
    pb.scale = float("nan")
    assert fwd_status(pb) == 2


def test_invalid_rank_ranges():
    pb = problem()
    assert fwd_status(pb, rb=-1, re_=2) == 2
    assert fwd_status(pb, rb=2, re_=2) == 2
    assert fwd_status(pb, rb=0, re_=5) == 2


def test_null_pointers():
    lib = ra.library()
    assert lib.ra_forward(None, 0, 1, None, None, None, None, None, None, 0, None, None) == 1
    pb = problem()
    seqs = [fake_seq() for _ in range(4)]
    seqs[2] = None
    assert fwd_status(pb, seqs=seqs) == 1
    seqs = [fake_seq() for _ in range(4)]
    seqs[0].ptr = None
    assert fwd_status(pb, seqs=seqs) == 1
    assert fwd_status(pb, lse=None) == 1


def test_misaligned_pointers_and_strides():
    pb = problem()
    seqs = [fake_seq() for _ in range(4)]
    seqs[1] = fake_seq(ptr=0x10008)
    assert fwd_status(pb, seqs=seqs) == 5
    seqs = [fake_seq() for _ in range(4)]
    seqs[3] = fake_seq(s_tok=513)  # 1026 bytes: not a multiple of 16
    assert fwd_status(pb, seqs=seqs) == 5
    seqs = [fake_seq() for _ in range(4)]
    seqs[0] = fake_seq(s_head=-64)
    assert fwd_status(pb, seqs=seqs) == 2
    assert fwd_status(pb, lse=0x20002) == 5


def test_copy_mode_requires_one_rank_and_workspace():
    pb = problem()
    fake_stream = ctypes.c_void_p(0x1234)
    assert fwd_status(pb, rb=0, re_=2, copy=fake_stream) == 2
    assert fwd_status(pb, rb=1, re_=2, copy=fake_stream, ws=None) == 4
    need = ra.workspace_bytes(pb, 1, 2, True, False)
    assert fwd_status(pb, rb=1, re_=2, copy=fake_stream, ws=0x100000, ws_bytes=need - 1) == 4
    assert fwd_status(pb, rb=1, re_=2, copy=fake_stream, ws=0x100010, ws_bytes=need) == 5


def test_backward_validation():
    lib = ra.library()
    pb = problem()
    s = [fake_seq() for _ in range(8)]
    args = lambda ws, nbytes, lse=0x20000: (ctypes.byref(pb), 0, 4, *[ra._ref(x) for x in s[:5]], lse,
                                            *[ra._ref(x) for x in s[5:]], ws, nbytes, None)
    assert lib.ra_backward(*args(None, 0)) == 4
    need = ra.workspace_bytes(pb, 0, 4, False, 2)
    assert lib.ra_backward(*args(0x100000, need - 4)) == 4
    assert lib.ra_backward(*args(0x100000, need, lse=None)) == 1
    s[6] = None
    assert lib.ra_backward(*args(0x100000, need)) == 1
    # the bf16 dK/dV walk addresses a 64-row Q / dO tile with 32-bit offsets;
    # checked before the workspace, so these fail without launching anything
    for idx in (0, 4):
        s = [fake_seq() for _ in range(8)]
        s[idx] = fake_seq(s_tok=1 << 24)
        assert lib.ra_backward(*args(None, 0)) == 3
    s = [fake_seq() for _ in range(8)]
    s[0] = fake_seq(s_tok=(1 << 24) - 8)
    assert lib.ra_backward(*args(None, 0)) == 4


def test_merge_and_layout_copy_validation():
    lib = ra.library()
    p = 0x10000
    assert lib.ra_merge_lse(4, 64, None, p, p, p, p, p, None) == 1
    assert lib.ra_merge_lse(-1, 64, p, p, p, p, p, p, None) == 2
    assert lib.ra_merge_lse(4, 0, p, p, p, p, p, p, None) == 2
    assert lib.ra_merge_lse(4, 2048, p, p, p, p, p, p, None) == 2
    assert lib.ra_merge_lse(4, 64, p + 8, p, p, p, p, p, None) == 5
    assert lib.ra_merge_lse(4, 64, p, p + 2, p, p, p, p, None) == 5
    pb = problem()
    assert lib.ra_layout_copy(ctypes.byref(pb), None, p, 0, None) == 1
    assert lib.ra_layout_copy(ctypes.byref(pb), p + 4, p, 0, None) == 5
    assert lib.ra_layout_copy(None, p, p, 0, None) == 1


def test_linear_and_layer_norm_validation():
    """Argument checks only: every call here fails validation, so nothing is
    launched."""
    lib = ra.library()
    p = 0x10000
    # n must be a multiple of 128, k of 64; m >= 1
    assert lib.ra_linear(64, 100, 64, p, 64, p, 64, None, None, 0, 0, p, 128, 1, None) == 2
    assert lib.ra_linear(64, 128, 96, p, 96, p, 96, None, None, 0, 0, p, 128, 1, None) == 2
    assert lib.ra_linear(0, 128, 64, p, 64, p, 64, None, None, 0, 0, p, 128, 1, None) == 2
    assert lib.ra_linear(64, 128, 64, p, 32, p, 64, None, None, 0, 0, p, 128, 1, None) == 2  # lda < k
    assert lib.ra_linear(64, 128, 64, None, 64, p, 64, None, None, 0, 0, p, 128, 1, None) == 1
    assert lib.ra_linear(64, 128, 64, p + 2, 64, p, 64, None, None, 0, 0, p, 128, 1, None) == 5
    assert lib.ra_linear(64, 128, 64, p, 68, p, 64, None, None, 0, 0, p, 128, 1, None) == 5  # row stride
    assert lib.ra_layer_norm(4, 8193, p, p, p, 0.0, p, None) == 2
    assert lib.ra_layer_norm(4, 0, p, p, p, 0.0, p, None) == 2
    assert lib.ra_layer_norm(4, 64, None, p, p, 0.0, p, None) == 1
    assert lib.ra_layer_norm(4, 64, p, p, p, float("nan"), p, None) == 2


def test_bpt_validation_and_workspace():
    br, dm, dff = 1024, 4096, 16384
    pb = ra.BptProblem(32768, dm, dff, br, 0.0)
    assert ra.bpt_workspace_bytes(pb) == br * dm * 4 + br * dm * 2 + br * dff * 2
    assert ra.bpt_workspace_bytes(ra.BptProblem(100, dm, dff, br, 0.0)) == 100 * (dm * 4 + dm * 2 + dff * 2)
    for bad in (ra.BptProblem(32768, 4000, dff, br, 0.0), ra.BptProblem(32768, dm, 1000, br, 0.0),
                ra.BptProblem(0, dm, dff, br, 0.0), ra.BptProblem(32768, 16384, dff, br, 0.0)):
        assert ra.bpt_workspace_bytes(bad) == 0
    lib = ra.library()
    w = ra.BptWeights(*([0x10000] * 10))
    p = 0x20000
    assert lib.ra_bpt_ffn(ctypes.byref(pb), p, p, ctypes.byref(w), p, None, 0, None) == 4  # no workspace
    w0 = ra.BptWeights(*([0x10000] * 9 + [0]))
    assert lib.ra_bpt_ffn(ctypes.byref(pb), p, p, ctypes.byref(w0), p, p, 1 << 40, None) == 1
    assert lib.ra_bpt_ffn(ctypes.byref(ra.BptProblem(32768, 4000, dff, br, 0.0)), p, p, ctypes.byref(w), p, p,
                          1 << 40, None) == 2


def test_noalloc_backward_rejects_problems_beyond_its_scratch():
    """ra_backward_noalloc keeps 8 bytes per query row in a static array of
    ra_backward_noalloc_max_bytes(); a larger problem returns RA_ERR_SCRATCH,
    and invalid arguments their usual codes, before anything is launched."""
    lib = ra.library()
    cap = ra.backward_noalloc_max_bytes()
    assert cap == 64 << 20
    s = [fake_seq() for _ in range(8)]

    def call(pb, lse=0x20000, seqs=s):
        return lib.ra_backward_noalloc(ctypes.byref(pb), 0, pb.ring_size, *[ra._ref(x) for x in seqs[:5]], lse,
                                       *[ra._ref(x) for x in seqs[5:]], None)
    big = problem(d=128, P=8, Bb=65536, H=32)  # 8 * 32 * 65536 rows * 8 B = 128 MiB
    assert ra.workspace_bytes(big, 0, 8, False, 2) > cap
    assert call(big) == 7
    assert "static scratch" in ra.status_string(7)
    assert call(problem(), lse=None) == 1
    bad = [fake_seq() for _ in range(8)]
    bad[6] = fake_seq(ptr=0x10008)
    assert call(problem(), seqs=bad) == 5
    pb = problem()
    pb.head_dim = 96
    assert call(pb) == 3


def test_binding_tells_the_library_the_size_of_the_callers_workspace(monkeypatch):
    """The workspace size decides the mode (the backward stores dS only in a
    buffer of the full size, the forward splits only in one of the split
    size), so the binding must pass the size of the buffer it was given,
    never the size it would have allocated. The raw calls are captured here;
    nothing is launched."""
    torch = pytest.importorskip("torch")
    seen = {}
    monkeypatch.setattr(ra, "_stream_handle", lambda s: None)
    monkeypatch.setattr(ra, "backward_raw", lambda *a: seen.__setitem__("bwd", a[-2]))
    monkeypatch.setattr(ra, "forward_raw", lambda *a: seen.__setitem__("fwd", (a[-4], a[-3])))
    B, H, d, P, Bb = 1, 2, 64, 4, 128
    L = P * Bb
    q, k, v, o, do = (torch.zeros(B, L, H, d, dtype=torch.bfloat16) for _ in range(5))
    lse = torch.zeros(P, B, H, Bb)
    pb = ra.make_problem(B, H, d, P, Bb, "striped", True, ra.BF16, None, kv_heads=H)
    full = ra.workspace_bytes(pb, 0, P, False, True)
    small = ra.workspace_bytes(pb, 0, P, False, 2)
    assert 0 < small < full
    ra.attention_backward(q, k, v, o, do, lse, P, "striped", True)
    assert seen["bwd"] == full
    ra.attention_backward(q, k, v, o, do, lse, P, "striped", True,
                          workspace=torch.empty(small, dtype=torch.uint8))
    assert seen["bwd"] == small
    ra.attention_backward(q, k, v, o, do, lse, P, "striped", True,
                          workspace=torch.empty(small // 4 + 8, dtype=torch.float32))
    assert seen["bwd"] == (small // 4 + 8) * 4
    # forward, one rank of a ring too short to fill the GPU: the split size
    pf = ra.make_problem(B, H, d, 3, 300, "striped", True, ra.BF16, None, kv_heads=H)
    need = ra.workspace_bytes(pf, 2, 3, False, False)
    q3, k3, v3 = (torch.zeros(B, 900, H, d, dtype=torch.bfloat16) for _ in range(3))
    ra.attention_forward(q3, k3, v3, 3, "striped", True, rank_range=(2, 3))
    assert seen["fwd"][1] == need
    ra.attention_forward(q3, k3, v3, 3, "striped", True, rank_range=(2, 3),
                         workspace=torch.empty(need // 2, dtype=torch.uint8))
    assert seen["fwd"][1] == need // 2  # too small to split: the library runs one unsplit launch
    ra.attention_forward(q3, k3, v3, 3, "striped", True, rank_range=(2, 3), split=False)
    assert seen["fwd"] == (None, 0)


def test_binding_refuses_buffers_the_library_cannot_check():
    """Shapes, element types and contiguity the C ABI cannot see (it takes
    pointers and strides) are checked by the binding before any pointer is
    handed over; each bad argument raises ValueError. CPU tensors: nothing
    reaches the library."""
    torch = pytest.importorskip("torch")
    bf, f32 = torch.bfloat16, torch.float32
    B, L, H, d, P = 1, 512, 4, 64, 4
    Bb = L // P
    q = torch.zeros(B, L, H, d, dtype=bf)
    k = torch.zeros(B, L, 2, d, dtype=bf)
    lse = torch.zeros(P, B, H, Bb)
    z = lambda *s, dt=bf: torch.zeros(*s, dtype=dt)  # noqa: E731
    bad = [
        lambda: ra.attention_forward(z(B, 510, H, d), z(B, 510, 2, d), z(B, 510, 2, d), P),      # 510 % 4
        lambda: ra.attention_forward(q, k, k, P, rank_range=(2, 5)),                             # past the ring
        lambda: ra.attention_forward(q, k, k, P, rank_range=(2, 2)),                             # empty
        lambda: ra.attention_forward(q, k, z(B, L, 3, d), P),                                    # v != k
        lambda: ra.attention_forward(q, z(B, L, 3, d), z(B, L, 3, d), P),                        # 3 does not divide 4
        lambda: ra.attention_forward(q, k.float(), k, P),                                        # mixed dtypes
        lambda: ra.attention_forward(z(B, 200, H, d), k, k, P, rank_range=(0, 2)),              # rows of 2 ranks: 256
        lambda: ra.attention_forward(q, k, k, P, lse=torch.zeros(P - 1, B, H, Bb)),              # lse too small
        lambda: ra.attention_forward(q, k, k, P, lse=torch.zeros(P, B, H, Bb, dtype=torch.float64)),
        lambda: ra.attention_forward(q, k, k, P, out=z(B, L, H, d, dt=f32)),                     # out dtype
        lambda: ra.attention_backward(q, k, k, z(B, L, H, 32), q, lse, P),                       # o shape
        lambda: ra.attention_backward(q, k, k, q, q, lse[:2], P),                                # lse rows
        lambda: ra.attention_backward(q, k, k, q, q, torch.zeros(P, B, H, 2 * Bb)[..., ::2], P),   # strided lse
        lambda: ra.attention_backward(q[:, :256], k, k, q[:, :256], q[:, :256], lse[:2], P, rank_range=(0, 2)),
        lambda: ra.merge_lse(z(8, 64, dt=f32).t(), z(64, dt=f32), z(64, 8, dt=f32), z(64, dt=f32)),
        lambda: ra.merge_lse(z(64, 8, dt=f32), z(63, dt=f32), z(64, 8, dt=f32), z(64, dt=f32)),
        lambda: ra.merge_lse(z(64, 8, dt=f32), z(64, dt=f32), z(64, 8), z(64, dt=f32)),
        lambda: ra.layout_copy(q.transpose(1, 2), P, "striped"),                                 # not contiguous
        lambda: ra.layout_copy(z(B, 510, H, d), P, "striped"),
        lambda: ra.linear(z(16, 64), z(32, 48)),                                                 # k mismatch
        lambda: ra.linear(z(16, 64), z(32, 64), bias=z(32)),                                     # bias dtype
        lambda: ra.linear(z(16, 64), z(32, 64), residual=z(16, 32, dt=f32)),                     # residual dtype
        lambda: ra.linear(z(16, 64), z(32, 64), out=z(16, 32, dt=f32)),                          # out dtype
        lambda: ra.layer_norm(z(16, 64, dt=f32), z(63, dt=f32), z(64, dt=f32)),
        lambda: ra.layer_norm(z(16, 64), z(64, dt=f32), z(64, dt=f32)),                          # z dtype
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    dm, dff = 128, 256
    w = {n: z(dm, dt=f32) for n in ra.BPT_WEIGHT_NAMES}
    w.update(w_o=z(dm, dm), w_1=z(dff, dm), w_2=z(dm, dff), b_1=z(dff, dt=f32))
    for name, wrong in (("w_2", z(dff, dm)), ("b_1", z(dm, dt=f32)), ("ln1_g", z(dm)), ("w_o", z(dm, dm, dt=f32))):
        ww = dict(w, **{name: wrong})
        with pytest.raises(ValueError):
            ra.bpt_ffn(z(64, dm), z(64, dm), ww, 32)
