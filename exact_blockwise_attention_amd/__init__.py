"""exact_blockwise_attention_amd — Python binding of libra.so (gfx950).

A thin ctypes layer over the C ABI declared in include/ra.h: it marshals
arguments (device pointers, strides, stream handles) and nothing else; every
step of the computation runs in the HIP kernels behind the ABI. PyTorch is
used only to hold device memory and to name streams. There is no CPU
fallback: if the library is missing or fails to load, every call raises.

Low level:  Problem, Seq, forward_raw, backward_raw, merge_lse_raw,
            layout_copy_raw, workspace_bytes, linear_raw, layer_norm_raw,
            bpt_ffn_raw (same names and meaning as the C functions).
High level: attention_forward / attention_backward take original-order
            [B, L, H, d] torch tensors (K and V may have fewer heads than Q:
            grouped-query attention) and allocate outputs/workspaces with
            torch; linear, layer_norm, bpt_ffn and bpt_layer cover the
            Blockwise Parallel Transformer layer around attention.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LAYOUT_CONTIGUOUS", "LAYOUT_STRIPED", "F32", "BF16", "Problem", "Seq", "RaError",
    "library", "library_path", "workspace_bytes", "forward_raw", "backward_raw", "merge_lse_raw",
    "layout_copy_raw", "status_string", "abi_version", "seq_original", "seq_blocked", "LAYOUTS",
    "attention_forward", "attention_backward", "merge_lse", "layout_copy", "EXPORTED_FUNCTIONS",
    "BptProblem", "BptWeights", "linear_raw", "layer_norm_raw", "bpt_ffn_raw", "bpt_workspace_bytes",
    "linear", "layer_norm", "bpt_ffn", "bpt_layer", "BPT_WEIGHT_NAMES",
]

LAYOUT_CONTIGUOUS = 0
LAYOUT_STRIPED = 1
LAYOUT_ZIGZAG = 2
LAYOUTS = {"contiguous": LAYOUT_CONTIGUOUS, "striped": LAYOUT_STRIPED, "zigzag": LAYOUT_ZIGZAG}
F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libra.so")

EXPORTED_FUNCTIONS = (
    "ra_workspace_bytes", "ra_forward", "ra_backward", "ra_backward_stage", "ra_merge_lse", "ra_layout_copy",
    "ra_linear", "ra_layer_norm", "ra_bpt_workspace_bytes", "ra_bpt_ffn", "ra_status_string", "ra_abi_version",
    "ra_backward_noalloc", "ra_backward_noalloc_max_bytes",
)


class RaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("ring_size", ctypes.c_int32), ("block_len", ctypes.c_int64), ("layout", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
    ]


class Seq(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p), ("s_blk", ctypes.c_int64), ("s_batch", ctypes.c_int64),
        ("s_tok", ctypes.c_int64), ("s_head", ctypes.c_int64),
    ]


class BptProblem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("block_rows", ctypes.c_int64), ("ln_eps", ctypes.c_float)]


BPT_WEIGHT_NAMES = ("w_o", "b_o", "ln1_g", "ln1_b", "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


class BptWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BPT_WEIGHT_NAMES]


_lib = None


def library():
    """Load libra.so once; raise loudly if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with `python -m exact_blockwise_attention_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(library_path)
    P, S, vp, i32, i64, sz = (ctypes.POINTER(Problem), ctypes.POINTER(Seq), ctypes.c_void_p,
                              ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t)
    lib.ra_workspace_bytes.argtypes = [P, i32, i32, i32, i32]
    lib.ra_workspace_bytes.restype = sz
    lib.ra_forward.argtypes = [P, i32, i32, S, S, S, S, vp, vp, sz, vp, vp]
    lib.ra_forward.restype = i32
    lib.ra_backward.argtypes = [P, i32, i32, S, S, S, S, S, vp, S, S, S, vp, sz, vp]
    lib.ra_backward.restype = i32
    lib.ra_backward_stage.argtypes = [i32, P, i32, i32, S, S, S, S, S, vp, S, S, S, vp, sz, vp]
    lib.ra_backward_stage.restype = i32
    lib.ra_backward_noalloc.argtypes = [P, i32, i32, S, S, S, S, S, vp, S, S, S, vp]
    lib.ra_backward_noalloc.restype = i32
    lib.ra_backward_noalloc_max_bytes.argtypes = []
    lib.ra_backward_noalloc_max_bytes.restype = sz
    lib.ra_merge_lse.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_merge_lse.restype = i32
    lib.ra_layout_copy.argtypes = [P, vp, vp, i32, vp]
    lib.ra_layout_copy.restype = i32
    lib.ra_linear.argtypes = [i64, i32, i32, vp, i64, vp, i64, vp, vp, i64, i32, vp, i64, i32, vp]
    lib.ra_linear.restype = i32
    lib.ra_layer_norm.argtypes = [i64, i32, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.ra_layer_norm.restype = i32
    BP, BW = ctypes.POINTER(BptProblem), ctypes.POINTER(BptWeights)
    lib.ra_bpt_workspace_bytes.argtypes = [BP]
    lib.ra_bpt_workspace_bytes.restype = sz
    lib.ra_bpt_ffn.argtypes = [BP, vp, vp, BW, vp, vp, sz, vp]
    lib.ra_bpt_ffn.restype = i32
    lib.ra_status_string.argtypes = [i32]
    lib.ra_status_string.restype = ctypes.c_char_p
    lib.ra_abi_version.argtypes = []
    lib.ra_abi_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().ra_status_string(int(status)).decode()


def abi_version() -> int:
    return int(library().ra_abi_version())


def _check(fn, status):
    if status != 0:
        raise RaError(fn, status)


def _ref(x):
    return None if x is None else ctypes.byref(x)


def workspace_bytes(pb: Problem, rank_begin: int, rank_end: int, use_copy_stream: bool, backward) -> int:
    """backward: 0 forward; 1 (True) the backward's full workspace (bf16: dS
    stored once); 2 the backward's minimum (dQ recomputes S and dP)."""
    return int(library().ra_workspace_bytes(ctypes.byref(pb), rank_begin, rank_end,
                                            int(bool(use_copy_stream)), int(backward)))


def forward_raw(pb, rank_begin, rank_end, q, k, v, o, lse_ptr, ws_ptr, ws_bytes, compute, copy):
    """ra_forward with already-marshalled arguments (Seq structs, ints)."""
    st = library().ra_forward(ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v), _ref(o),
                              lse_ptr, ws_ptr, ws_bytes, compute, copy)
    _check("ra_forward", st)


def backward_raw(pb, rank_begin, rank_end, q, k, v, o, do, lse_ptr, dq, dk, dv, ws_ptr, ws_bytes, compute):
    st = library().ra_backward(ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v), _ref(o),
                               _ref(do), lse_ptr, _ref(dq), _ref(dk), _ref(dv), ws_ptr, ws_bytes, compute)
    _check("ra_backward", st)


def backward_noalloc_raw(pb, rank_begin, rank_end, q, k, v, o, do, lse_ptr, dq, dk, dv, compute):
    """ra_backward_noalloc: ra_backward with the library's static scratch
    instead of a workspace."""
    st = library().ra_backward_noalloc(ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v), _ref(o),
                                       _ref(do), lse_ptr, _ref(dq), _ref(dk), _ref(dv), compute)
    _check("ra_backward_noalloc", st)


def backward_noalloc_max_bytes() -> int:
    return int(library().ra_backward_noalloc_max_bytes())


def backward_stage_raw(stage, pb, rank_begin, rank_end, q, k, v, o, do, lse_ptr, dq, dk, dv, ws_ptr, ws_bytes,
                       compute):
    st = library().ra_backward_stage(stage, ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v),
                                     _ref(o), _ref(do), lse_ptr, _ref(dq), _ref(dk), _ref(dv), ws_ptr, ws_bytes,
                                     compute)
    _check("ra_backward_stage", st)


def merge_lse_raw(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out, stream):
    st = library().ra_merge_lse(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, lse_out, stream)
    _check("ra_merge_lse", st)


def layout_copy_raw(pb, src, dst, inverse, stream):
    st = library().ra_layout_copy(ctypes.byref(pb), src, dst, int(bool(inverse)), stream)
    _check("ra_layout_copy", st)


def linear_raw(m, n, k, a, lda, w, ldw, bias, residual, ldr, gelu, out, ldo, out_f32, stream):
    st = library().ra_linear(m, n, k, a, lda, w, ldw, bias, residual, ldr, int(bool(gelu)), out, ldo,
                             int(bool(out_f32)), stream)
    _check("ra_linear", st)


def layer_norm_raw(rows, d, z, gamma, beta, eps, out, stream):
    st = library().ra_layer_norm(rows, d, z, gamma, beta, float(eps), out, stream)
    _check("ra_layer_norm", st)


def bpt_workspace_bytes(pb: BptProblem) -> int:
    return int(library().ra_bpt_workspace_bytes(ctypes.byref(pb)))


def bpt_ffn_raw(pb, attn, x, wts, out, ws_ptr, ws_bytes, stream):
    st = library().ra_bpt_ffn(ctypes.byref(pb), attn, x, ctypes.byref(wts), out, ws_ptr, ws_bytes, stream)
    _check("ra_bpt_ffn", st)


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch  # noqa: WPS433 (torch is only plumbing: memory and streams)
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def seq_original(t, ring_size: int, layout: str, block_offset: int = 0) -> Seq:
    """Describe an original-order [B, L, H, d] tensor as ring blocks.

    ``block_offset`` shifts block 0 to block ``block_offset`` (so that index
    rank - rank_begin addresses rank's block in a full-sequence tensor).
    """
    B, L, H, d = t.shape
    sb, sl, sh, se = t.stride()
    if se != 1:
        raise ValueError("features must be contiguous")
    if L % ring_size:
        raise ValueError("sequence must split into equal blocks")
    Bb = L // ring_size
    if layout == "zigzag":
        raise ValueError("a zigzag block is not a strided slice of the original order: use blocked tensors")
    if layout == "striped":
        s_blk, s_tok = sl, ring_size * sl
    else:
        s_blk, s_tok = Bb * sl, sl
    ptr = t.data_ptr() + block_offset * s_blk * t.element_size()
    return Seq(ptr, s_blk, sb, s_tok, sh)


def seq_blocked(t, block_offset: int = 0) -> Seq:
    """Describe a blocked [P, B, Bb, H, d] tensor (block ``block_offset`` first)."""
    P, B, Bb, H, d = t.shape
    s = t.stride()
    if s[4] != 1:
        raise ValueError("features must be contiguous")
    return Seq(t.data_ptr() + block_offset * s[0] * t.element_size(), s[0], s[1], s[2], s[3])


def _seq_for(t, P, layout, block_offset=0):
    """Ring-block description of an original-order tensor; for the zigzag
    layout a blocked copy (made with the library's layout copy) is described
    instead and returned alongside, so that the caller can keep it alive or
    copy results back."""
    if layout == "zigzag":
        tb = layout_copy(t, P, layout)
        return seq_blocked(tb, block_offset), tb
    return seq_original(t, P, layout, block_offset=block_offset), None


def make_problem(B, H, d, P, Bb, layout, causal, dtype_code, scale=None, kv_heads=0) -> Problem:
    """kv_heads: heads of K and V (0: the same as H)."""
    return Problem(B, H, d, P, Bb, LAYOUTS[layout], int(bool(causal)),
                   float(scale) if scale else 0.0, dtype_code, int(kv_heads))


def _nbytes(t) -> int:
    """Bytes of a workspace tensor, as the library is told them."""
    return int(t.numel()) * int(t.element_size())


# The library sees pointers and strides only: it cannot tell a buffer that is
# too small or of another element type. These checks run before any pointer
# is handed over and raise ValueError.
def _expect(t, name, shape=None, dtype=None, device=None, contiguous=False, dims=None):
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {dims}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_attention_inputs(q, k, v, P, rank_range):
    """q [B, L or nr*Bb, H, d], k and v [B, L, Hk, d] of one dtype and device,
    Hk dividing H, L a multiple of P, 0 <= rank_begin < rank_end <= P."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, n, dims=4, dtype=q.dtype, device=q.device)
    _expect(v, "v", shape=k.shape)
    B, L, Hk, d = k.shape
    if P < 1 or L % P:
        raise ValueError(f"sequence length {L} must split into {P} equal blocks")
    rb, re = (0, P) if rank_range is None else rank_range
    if not 0 <= rb < re <= P:
        raise ValueError(f"rank range [{rb}, {re}) outside the ring of {P}")
    if q.shape[0] != B or q.shape[3] != d or q.shape[1] not in (L, (re - rb) * (L // P)):
        raise ValueError(f"q: shape {tuple(q.shape)} does not match k {tuple(k.shape)} and the rank range")
    if q.shape[2] % Hk:
        raise ValueError(f"{Hk} K/V heads must divide {q.shape[2]} query heads")
    return rb, re


def attention_forward(q, k, v, ring_size: int, layout: str = "contiguous", causal: bool = False,
                      scale=None, rank_range=None, copy_stream=None, out=None, lse=None, workspace=None,
                      split=True):
    """Blockwise ring attention forward on original-order [B, L, H, d] tensors.

    k, v: the whole sequence, [B, L, Hk, d] with Hk dividing H (query head h
    reads K/V head h // (H / Hk)). q (and ``out``) hold either the whole sequence
    ([B, L, H, d], only the rows of the ranks in ``rank_range`` are read /
    written) or just those ranks' rows ([B, nr*Bb, H, d], each rank's block
    contiguous in its local row order). Returns (o, lse) with lse fp32
    [nr, B, H, Bb] in local row order. A non-None ``copy_stream`` selects the
    double-buffered receive mode (single rank). Without it, a single rank
    whose query tiles cannot fill the GPU runs its ring steps as parallel runs
    merged by log-sum-exp (the library does so when it is given the workspace
    ra_workspace_bytes asks for); ``split=False`` passes no workspace, so the
    whole ring runs in one unsplit launch.
    """
    torch = _torch()
    P = ring_size
    rb, re = _check_attention_inputs(q, k, v, P, rank_range)
    B, L, Hk, d = k.shape
    H = q.shape[2]
    Bb = L // P
    nr = re - rb
    code = _dtype_code(q)
    pb = make_problem(B, H, d, P, Bb, layout, causal, code, scale, kv_heads=Hk)
    if out is not None:
        _expect(out, "out", shape=q.shape, dtype=q.dtype, device=q.device)
    if lse is not None:
        _expect(lse, "lse", shape=(nr, B, H, Bb), dtype=torch.float32, device=q.device, contiguous=True)
    if workspace is not None:
        _expect(workspace, "workspace", device=q.device, contiguous=True)
    if out is None:
        # rows of ranks outside the range are never written: zero them
        out = torch.zeros_like(q) if (q.shape[1] == L and nr < P) else torch.empty_like(q)
    if lse is None:
        lse = torch.empty((nr, B, H, Bb), dtype=torch.float32, device=q.device)
    use_copy = copy_stream is not None
    need = workspace_bytes(pb, rb, re, use_copy, False) if (split or use_copy) else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    # the library is told the size of the buffer it is given, which decides the mode
    ws_ptr, ws_size = (workspace.data_ptr(), _nbytes(workspace)) if need else (None, 0)
    keep = []
    if q.shape[1] == L:
        qs, t_ = _seq_for(q, P, layout, rb)
        keep.append(t_)
    else:
        qs = _seq_rank_rows(q, nr, layout, P)
    ob = None
    if out.shape[1] == L:
        os_, ob = _seq_for(out, P, layout, rb)
    else:
        os_ = _seq_rank_rows(out, nr, layout, P)
    ks, kb = _seq_for(k, P, layout)
    vs, vb = _seq_for(v, P, layout)
    forward_raw(pb, rb, re, qs, ks, vs, os_,
                lse.data_ptr(), ws_ptr, ws_size, _stream_handle(None),
                _stream_handle(copy_stream) if use_copy else None)
    if ob is not None:  # zigzag: blocked result back to the original order
        out.copy_(layout_copy(ob, P, layout, inverse=True))
    return out, lse


def _seq_rank_rows(t, nr, layout, P):
    """[B, nr*Bb, H, d] holding only the ranks' rows, each rank's block
    contiguous and in local row order."""
    B, Lr, H, d = t.shape
    sb, sl, sh, se = t.stride()
    if se != 1:
        raise ValueError("features must be contiguous")
    Bb = Lr // nr
    return Seq(t.data_ptr(), Bb * sl, sb, sl, sh)


def attention_backward(q, k, v, o, do, lse, ring_size: int, layout: str = "contiguous",
                       causal: bool = False, scale=None, rank_range=None, workspace=None, noalloc=False):
    """Backward on original-order [B, L, H, d] tensors (k, v, dk, dv with
    Hk heads); returns (dq, dk, dv). ``noalloc`` calls ra_backward_noalloc,
    which takes no workspace (the library's static scratch instead)."""
    torch = _torch()
    P = ring_size
    rb, re = _check_attention_inputs(q, k, v, P, rank_range)
    B, L, Hk, d = k.shape
    H = q.shape[2]
    Bb = L // P
    _expect(q, "q", shape=(B, L, H, d))
    for t, n in ((o, "o"), (do, "do")):
        _expect(t, n, shape=q.shape, dtype=q.dtype, device=q.device)
    _expect(lse, "lse", shape=(re - rb, B, H, Bb), dtype=torch.float32, device=q.device, contiguous=True)
    if workspace is not None:
        _expect(workspace, "workspace", device=q.device, contiguous=True)
    code = _dtype_code(q)
    pb = make_problem(B, H, d, P, Bb, layout, causal, code, scale, kv_heads=Hk)
    dq = torch.zeros_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None and not noalloc:
        workspace = torch.empty(workspace_bytes(pb, rb, re, False, True), dtype=torch.uint8, device=q.device)
    (qs, _q), (os_, _o), (ds, _d) = (_seq_for(t, P, layout, rb) for t in (q, o, do))
    (ks, _k), (vs, _v) = (_seq_for(t, P, layout) for t in (k, v))
    (dqs, dqb), (dks, dkb), (dvs, dvb) = (_seq_for(dq, P, layout, rb), _seq_for(dk, P, layout),
                                          _seq_for(dv, P, layout))
    if noalloc:
        backward_noalloc_raw(pb, rb, re, qs, ks, vs, os_, ds, lse.data_ptr(), dqs, dks, dvs, _stream_handle(None))
    else:
        # a caller's smaller workspace (at least workspace_bytes(..., 2)) selects
        # the path that recomputes dQ instead of storing dS
        backward_raw(pb, rb, re, qs, ks, vs, os_, ds, lse.data_ptr(), dqs, dks, dvs,
                     workspace.data_ptr(), _nbytes(workspace), _stream_handle(None))
    if layout == "zigzag":  # blocked results back to the original order
        for t, tb in ((dq, dqb), (dk, dkb), (dv, dvb)):
            t.copy_(layout_copy(tb, P, layout, inverse=True))
    return dq, dk, dv


def merge_lse(o_a, lse_a, o_b, lse_b, out=None, lse_out=None):
    """fp32 [rows, d] / [rows] partial results -> merged (o, lse)."""
    torch = _torch()
    _expect(o_a, "o_a", dims=2, dtype=torch.float32, contiguous=True)
    rows, d = o_a.shape
    dev = o_a.device
    _expect(o_b, "o_b", shape=(rows, d), dtype=torch.float32, device=dev, contiguous=True)
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        _expect(t, n, shape=(rows,), dtype=torch.float32, device=dev, contiguous=True)
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    _expect(out, "out", shape=(rows, d), dtype=torch.float32, device=dev, contiguous=True)
    _expect(lse_out, "lse_out", shape=(rows,), dtype=torch.float32, device=dev, contiguous=True)
    merge_lse_raw(rows, d, o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                  out.data_ptr(), lse_out.data_ptr(), _stream_handle(None))
    return out, lse_out


def layout_copy(x, ring_size: int, layout: str, inverse: bool = False):
    """Original [B, L, H, d] -> blocked [P, B, Bb, H, d] (or back)."""
    torch = _torch()
    _expect(x, "x", dims=5 if inverse else 4, contiguous=True)
    if not inverse and (ring_size < 1 or x.shape[1] % ring_size):
        raise ValueError(f"sequence length {x.shape[1]} must split into {ring_size} equal blocks")
    if inverse:
        P, B, Bb, H, d = x.shape
        out = torch.empty((B, P * Bb, H, d), dtype=x.dtype, device=x.device)
    else:
        B, L, H, d = x.shape
        P, Bb = ring_size, L // ring_size
        out = torch.empty((P, B, Bb, H, d), dtype=x.dtype, device=x.device)
    pb = make_problem(B, H, d, P, Bb, layout, True, _dtype_code(x))
    layout_copy_raw(pb, x.data_ptr(), out.data_ptr(), inverse, _stream_handle(None))
    return out


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# ---------------------------------------------------------------- the BPT layer

def _ptr(t):
    return None if t is None else t.data_ptr()


def linear(x, w, bias=None, residual=None, gelu=False, out_f32=False, out=None):
    """x [m, k] bf16, w [n, k] bf16 (a linear layer's [out, in] weight) ->
    x w^T (+ bias) (+ residual) (then GELU), [m, n] fp32 or bf16."""
    torch = _torch()
    _expect(x, "x", dims=2, dtype=torch.bfloat16)
    m, k = x.shape
    dev = x.device
    _expect(w, "w", dims=2, dtype=torch.bfloat16, device=dev)
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError(f"w: shape {tuple(w.shape)} does not match x {tuple(x.shape)}")
    if bias is not None:
        _expect(bias, "bias", shape=(n,), dtype=torch.float32, device=dev, contiguous=True)
    if residual is not None:
        _expect(residual, "residual", shape=(m, n), dtype=torch.bfloat16, device=dev)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32 if out_f32 else torch.bfloat16, device=x.device)
    _expect(out, "out", shape=(m, n), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dev)
    for t, nme in ((x, "x"), (w, "w"), (out, "out")) + (((residual, "residual"),) if residual is not None else ()):
        if t.stride(1) != 1:
            raise ValueError(f"{nme}: rows must be contiguous")
    linear_raw(m, n, k, x.data_ptr(), x.stride(0), w.data_ptr(), w.stride(0), _ptr(bias), _ptr(residual),
               residual.stride(0) if residual is not None else 0, gelu, out.data_ptr(), out.stride(0), out_f32,
               _stream_handle(None))
    return out


def layer_norm(z, gamma, beta, eps=1e-5, out=None):
    """z [rows, d] fp32 -> bf16 layer norm over d."""
    torch = _torch()
    _expect(z, "z", dims=2, dtype=torch.float32, contiguous=True)
    rows, d = z.shape
    for t, n in ((gamma, "gamma"), (beta, "beta")):
        _expect(t, n, shape=(d,), dtype=torch.float32, device=z.device, contiguous=True)
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=z.device)
    _expect(out, "out", shape=(rows, d), dtype=torch.bfloat16, device=z.device, contiguous=True)
    layer_norm_raw(rows, d, z.data_ptr(), gamma.data_ptr(), beta.data_ptr(), eps, out.data_ptr(),
                   _stream_handle(None))
    return out


def bpt_ffn(attn, x, weights, block_rows, eps=1e-5, out=None, workspace=None):
    """The BPT layer after attention for rows [rows, d_model] (bf16): output
    projection, residual + LN1, feedforward network, residual + LN2, one
    block of ``block_rows`` rows at a time. ``weights``: dict of
    BPT_WEIGHT_NAMES tensors (weights bf16 [out, in], the rest fp32)."""
    torch = _torch()
    _expect(x, "x", dims=2, dtype=torch.bfloat16, contiguous=True)
    rows, dm = x.shape
    dev = x.device
    _expect(attn, "attn", shape=(rows, dm), dtype=torch.bfloat16, device=dev, contiguous=True)
    dff = weights["w_1"].shape[0]
    shapes = {"w_o": (dm, dm), "w_1": (dff, dm), "w_2": (dm, dff), "b_1": (dff,)}
    for n in BPT_WEIGHT_NAMES:
        _expect(weights[n], n, shape=shapes.get(n, (dm,)), dtype=torch.bfloat16 if n.startswith("w_") else torch.float32,
                device=dev, contiguous=True)
    if out is not None:
        _expect(out, "out", shape=(rows, dm), dtype=torch.bfloat16, device=dev, contiguous=True)
    if workspace is not None:
        _expect(workspace, "workspace", device=dev, contiguous=True)
    pb = BptProblem(rows, dm, dff, block_rows, eps)
    wts = BptWeights(*(weights[n].data_ptr() for n in BPT_WEIGHT_NAMES))
    need = bpt_workspace_bytes(pb)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty_like(x)
    bpt_ffn_raw(pb, attn.data_ptr(), x.data_ptr(), wts, out.data_ptr(), workspace.data_ptr(), _nbytes(workspace),
                _stream_handle(None))
    return out


def bpt_layer(x, weights, n_heads, ring_size, block_rows, causal=False, layout="contiguous"):
    """The whole layer on x [B, L, d_model] (bf16) with library calls only:
    Q, K, V projections (ra_linear), ring attention over ``ring_size``
    blocks (ra_forward), then bpt_ffn. ``weights`` also holds w_q, b_q,
    w_k, b_k, w_v, b_v."""
    B, L, dm = x.shape
    x2 = x.reshape(B * L, dm)
    q, k, v = (linear(x2, weights[f"w_{n}"], weights[f"b_{n}"]).reshape(B, L, n_heads, dm // n_heads)
               for n in "qkv")
    attn, _ = attention_forward(q, k, v, ring_size, layout, causal)
    return bpt_ffn(attn.reshape(B * L, dm), x2, weights, block_rows).reshape(B, L, dm)

