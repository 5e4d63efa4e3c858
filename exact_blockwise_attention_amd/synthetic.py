"""Seeded synthetic inputs and the workload table.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It holds no attention arithmetic: it draws i.i.d. N(0, 1) float32
samples from seeded numpy generators (one per chunk), rounds them to bfloat16
bit patterns when a workload is bf16, and widens bit patterns back to floats
so that both sides see exactly the same values.

Seeding: the tensor, flattened in its [B, L, H, d] (original token order)
layout, is cut into chunks of 2**22 elements; chunk c is drawn with
``standard_normal(dtype=float32)`` from
``numpy.random.Generator(PCG64(SeedSequence([workload_id, tensor_id, c])))``
with tensor ids Q=0, K=1, V=2, dO=3. Chunks are independent, so they are drawn
(and rounded) on several host threads.

The Blockwise Parallel Transformer layer adds its input x, an attention
output, and its parameters (ids from 10 on). Weights [out, in] are the N(0, 1)
draws scaled by 1/sqrt(in) and rounded to bfloat16, biases 0.02 N(0, 1), layer
norm gains 1 + 0.1 N(0, 1) and offsets 0.1 N(0, 1), all fp32 apart from the
weights: a scale that keeps activations of order one through the layer.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "x": 10, "attn": 11,
              "w_q": 12, "b_q": 13, "w_k": 14, "b_k": 15, "w_v": 16, "b_v": 17, "w_o": 18, "b_o": 19,
              "ln1_g": 20, "ln1_b": 21, "w_1": 22, "b_1": 23, "w_2": 24, "b_2": 25, "ln2_g": 26, "ln2_b": 27}


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, ring size, layout and precision.

    ``ring_size`` P splits the sequence of ``seq_len`` tokens into P equal
    blocks of ``block_len`` tokens (the ring of P devices). ``q_ranks`` is the
    half-open range of ranks whose query blocks are computed: the whole ring
    for the whole-sequence workloads, a single rank for one device's share.
    """

    wid: int
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    ring_size: int
    causal: bool
    layouts: tuple
    dtype: str  # "f32" or "bf16"
    passes: tuple  # ("fwd",) or ("fwd", "bwd")
    q_ranks: tuple | None = None  # None: all ranks
    prefetch: bool = False
    kv_heads: int = 0  # K/V heads (grouped-query attention); 0: the same as heads

    @property
    def block_len(self) -> int:
        return self.seq_len // self.ring_size


# The workloads: a tiny fp32 correctness case, a non-causal bf16 forward, a
# causal forward in every layout, one device's share of a 262,144-token
# 7B-shaped layer (H=32, d=128) with a prefetched side-stream KV receive, a
# causal striped forward+backward at 32,768 tokens, and the same with 8 K/V
# heads shared by the 32 query heads (grouped-query attention).
WORKLOADS = {
    1: Workload(1, "noncausal_f32_L1024_d64_P4", 1, 1, 1024, 64, 4, False,
                ("contiguous",), "f32", ("fwd",)),
    2: Workload(2, "noncausal_bf16_H8_L16384_d128_P8", 1, 8, 16384, 128, 8,
                False, ("contiguous",), "bf16", ("fwd",)),
    3: Workload(3, "causal_bf16_H32_L65536_d128_P16", 1, 32, 65536, 128, 16,
                True, ("contiguous", "striped"), "bf16", ("fwd",)),
    4: Workload(4, "share_causal_striped_bf16_H32_L262144_d128_P8_rank7", 1, 32,
                262144, 128, 8, True, ("striped",), "bf16", ("fwd",),
                q_ranks=(7, 8), prefetch=True),
    5: Workload(5, "causal_striped_bf16_H32_L32768_d128_P8_fwdbwd", 1, 32,
                32768, 128, 8, True, ("striped",), "bf16", ("fwd", "bwd")),
    6: Workload(6, "causal_striped_gqa_bf16_H32_KV8_L32768_d128_P8_fwdbwd", 1, 32,
                32768, 128, 8, True, ("striped",), "bf16", ("fwd", "bwd"), kv_heads=8),
}


def rng_for(workload_id: int, tensor_id: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tensor_id, chunk])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, fn):
    """Run fn(c, lo, hi) over the CHUNK-sized pieces of range(n), threaded."""
    pieces = [(c, lo, min(n, lo + CHUNK)) for c, lo in enumerate(range(0, n, CHUNK))]
    if len(pieces) <= 1:
        for p in pieces:
            fn(*p)
        return
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(lambda p: fn(*p), pieces))


def normal_f32(workload_id: int, tensor: str, shape) -> np.ndarray:
    """i.i.d. N(0,1) float32 array of ``shape`` for (workload, tensor)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    tid = TENSOR_IDS[tensor]

    def draw(c, lo, hi):
        out[lo:hi] = rng_for(workload_id, tid, c).standard_normal(size=hi - lo, dtype=np.float32)

    _chunked(n, draw)
    return out.reshape(shape)


def _round_bits(u: np.ndarray) -> np.ndarray:
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    out = t.astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) -> uint16 bits.

    NaN inputs map to a quiet NaN; the synthetic data never holds one.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)

    def rnd(c, lo, hi):
        out[lo:hi] = _round_bits(u[lo:hi])

    _chunked(u.size, rnd)
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_payload(workload_id: int, tensor: str, shape, dtype: str) -> np.ndarray:
    """The values the GPU receives: float32, or uint16 bfloat16 bit patterns."""
    x = normal_f32(workload_id, tensor, shape)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(payload: np.ndarray) -> np.ndarray:
    """Exact float64 widening of a payload (float32 or bf16 bit patterns)."""
    if payload.dtype == np.uint16:
        return bf16_bits_to_f32(payload).astype(np.float64)
    return payload.astype(np.float64)


def make_tensor(workload_id: int, tensor: str, shape, dtype: str):
    """Return (device_payload, exact_f64) for one input tensor.

    ``device_payload`` is a float32 array (dtype "f32") or the uint16 bf16 bit
    pattern array (dtype "bf16"); ``exact_f64`` is the same values widened to
    float64, for the oracle.
    """
    x = normal_f32(workload_id, tensor, shape)
    if dtype == "f32":
        return x, x.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def workload_shape(w: Workload, tensor: str = "q"):
    """[B, L, heads, d] of an input: K and V have the workload's K/V heads."""
    heads = (w.kv_heads or w.heads) if tensor in ("k", "v") else w.heads
    return (w.batch, w.seq_len, heads, w.head_dim)


def bpt_params(workload_id: int, d_model: int, d_ff: int) -> dict:
    """Parameters of a BPT layer: weights as bfloat16 bit patterns [out, in],
    the rest float32 (see the module docstring for the scales)."""
    shapes = {"q": (d_model, d_model), "k": (d_model, d_model), "v": (d_model, d_model),
              "o": (d_model, d_model), "1": (d_ff, d_model), "2": (d_model, d_ff)}
    p = {}
    for n, (o, i) in shapes.items():
        w = normal_f32(workload_id, f"w_{n}", (o, i)) * np.float32(1.0 / np.sqrt(i))
        p[f"w_{n}"] = f32_to_bf16_bits(w)
        p[f"b_{n}"] = normal_f32(workload_id, f"b_{n}", (o,)) * np.float32(0.02)
    for n in ("ln1", "ln2"):
        p[f"{n}_g"] = np.float32(1.0) + normal_f32(workload_id, f"{n}_g", (d_model,)) * np.float32(0.1)
        p[f"{n}_b"] = normal_f32(workload_id, f"{n}_b", (d_model,)) * np.float32(0.1)
    return p



# The Blockwise Parallel Transformer layer tail at the pages' 7B layer shape
# (hidden 4096 = 32 heads of 128, feedforward 4 x 4096), over a 32768-token
# sequence finished 4096 rows (one ring block of the forward+backward
# workload) at a time.
BPT_WORKLOAD = {"wid": 7, "name": "bpt_ffn_bf16_rows32768_d4096_ff16384_block4096", "rows": 32768,
                "d_model": 4096, "d_ff": 16384, "block_rows": 4096, "n_heads": 32}
