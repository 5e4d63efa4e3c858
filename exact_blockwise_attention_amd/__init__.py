"""exact_blockwise_attention_amd — Python binding of libra.so (gfx950).

A thin ctypes layer over the C ABI declared in include/ra.h: it marshals
arguments (device pointers, strides, stream handles) and nothing else; every
step of the computation runs in the HIP kernels behind the ABI. PyTorch is
used only to hold device memory and to name streams. There is no CPU
fallback: if the library is missing or fails to load, every call raises.

Low level:  Problem, Seq, forward_raw, backward_raw, merge_lse_raw,
            layout_copy_raw, workspace_bytes (same names and meaning as the
            C functions).
High level: attention_forward / attention_backward take original-order
            [B, L, H, d] torch tensors (K and V may have fewer heads than Q:
            grouped-query attention) and allocate outputs/workspaces with
            torch.
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
    "ra_status_string", "ra_abi_version",
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
    lib.ra_merge_lse.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_merge_lse.restype = i32
    lib.ra_layout_copy.argtypes = [P, vp, vp, i32, vp]
    lib.ra_layout_copy.restype = i32
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


def workspace_bytes(pb: Problem, rank_begin: int, rank_end: int, use_copy_stream: bool, backward: bool) -> int:
    return int(library().ra_workspace_bytes(ctypes.byref(pb), rank_begin, rank_end,
                                            int(bool(use_copy_stream)), int(bool(backward))))


def forward_raw(pb, rank_begin, rank_end, q, k, v, o, lse_ptr, ws_ptr, ws_bytes, compute, copy):
    """ra_forward with already-marshalled arguments (Seq structs, ints)."""
    st = library().ra_forward(ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v), _ref(o),
                              lse_ptr, ws_ptr, ws_bytes, compute, copy)
    _check("ra_forward", st)


def backward_raw(pb, rank_begin, rank_end, q, k, v, o, do, lse_ptr, dq, dk, dv, ws_ptr, ws_bytes, compute):
    st = library().ra_backward(ctypes.byref(pb), rank_begin, rank_end, _ref(q), _ref(k), _ref(v), _ref(o),
                               _ref(do), lse_ptr, _ref(dq), _ref(dk), _ref(dv), ws_ptr, ws_bytes, compute)
    _check("ra_backward", st)


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


def attention_forward(q, k, v, ring_size: int, layout: str = "contiguous", causal: bool = False,
                      scale=None, rank_range=None, copy_stream=None, out=None, lse=None, workspace=None):
    """Blockwise ring attention forward on original-order [B, L, H, d] tensors.

    k, v: the whole sequence, [B, L, Hk, d] with Hk dividing H (query head h
    reads K/V head h // (H / Hk)). q (and ``out``) hold either the whole sequence
    ([B, L, H, d], only the rows of the ranks in ``rank_range`` are read /
    written) or just those ranks' rows ([B, nr*Bb, H, d], each rank's block
    contiguous in its local row order). Returns (o, lse) with lse fp32
    [nr, B, H, Bb] in local row order. A non-None ``copy_stream`` selects the
    double-buffered receive mode (single rank).
    """
    torch = _torch()
    B, L, Hk, d = k.shape
    H = q.shape[2]
    P = ring_size
    Bb = L // P
    rb, re = (0, P) if rank_range is None else rank_range
    nr = re - rb
    code = _dtype_code(q)
    pb = make_problem(B, H, d, P, Bb, layout, causal, code, scale, kv_heads=Hk)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((nr, B, H, Bb), dtype=torch.float32, device=q.device)
    use_copy = copy_stream is not None
    need = workspace_bytes(pb, rb, re, use_copy, False)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
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
                lse.data_ptr(), workspace.data_ptr() if need else None, need, _stream_handle(None),
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
                       causal: bool = False, scale=None, rank_range=None, workspace=None):
    """Backward on original-order [B, L, H, d] tensors (k, v, dk, dv with
    Hk heads); returns (dq, dk, dv)."""
    torch = _torch()
    B, L, Hk, d = k.shape
    H = q.shape[2]
    P = ring_size
    Bb = L // P
    rb, re = (0, P) if rank_range is None else rank_range
    code = _dtype_code(q)
    pb = make_problem(B, H, d, P, Bb, layout, causal, code, scale, kv_heads=Hk)
    dq = torch.zeros_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    need = workspace_bytes(pb, rb, re, False, True)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    (qs, _q), (os_, _o), (ds, _d) = (_seq_for(t, P, layout, rb) for t in (q, o, do))
    (ks, _k), (vs, _v) = (_seq_for(t, P, layout) for t in (k, v))
    (dqs, dqb), (dks, dkb), (dvs, dvb) = (_seq_for(dq, P, layout, rb), _seq_for(dk, P, layout),
                                          _seq_for(dv, P, layout))
    backward_raw(pb, rb, re, qs, ks, vs, os_, ds, lse.data_ptr(), dqs, dks, dvs,
                 workspace.data_ptr(), need, _stream_handle(None))
    if layout == "zigzag":  # blocked results back to the original order
        for t, tb in ((dq, dqb), (dk, dkb), (dv, dvb)):
            t.copy_(layout_copy(tb, P, layout, inverse=True))
    return dq, dk, dv


def merge_lse(o_a, lse_a, o_b, lse_b, out=None, lse_out=None):
    """fp32 [rows, d] / [rows] partial results -> merged (o, lse)."""
    torch = _torch()
    rows, d = o_a.shape
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    merge_lse_raw(rows, d, o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                  out.data_ptr(), lse_out.data_ptr(), _stream_handle(None))
    return out, lse_out


def layout_copy(x, ring_size: int, layout: str, inverse: bool = False):
    """Original [B, L, H, d] -> blocked [P, B, Bb, H, d] (or back)."""
    torch = _torch()
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
