"""Helpers for the GPU parity tests: seeded inputs on the device, oracle
references on the host, and element-wise comparisons.

Inputs come from exact_blockwise_attention_amd.synthetic (the seeded
generator module shared with the oracle); references come from oracle/ only.
Nothing here computes attention itself.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

import oracle
from exact_blockwise_attention_amd import synthetic as syn

# Max-abs error bars against the float64 oracle, for the arithmetic (fp32
# accumulation). Outputs O, dQ, dK, dV are returned in the input dtype,
# rounded to nearest even, so a bfloat16 output may in addition differ from
# the exact value by half a bfloat16 spacing at that value (2^-8 |x| at most:
# 0.031 for |x| in [8, 16)); assert_output_close allows exactly that much
# more. lse is fp32 and gets the plain bar.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    seed: int
    B: int
    H: int
    L: int
    d: int
    P: int
    causal: bool
    layout: str
    dtype: str
    Hk: int = 0  # K/V heads (grouped-query attention); 0: the same as H

    @property
    def Bb(self):
        return self.L // self.P

    @property
    def kv_heads(self):
        return self.Hk or self.H

    @property
    def shape(self):
        return (self.B, self.L, self.H, self.d)

    def shape_of(self, name):
        return (self.B, self.L, self.kv_heads, self.d) if name in ("k", "v") else self.shape

    def __str__(self):
        kv = f" Hk={self.kv_heads}" if self.kv_heads != self.H else ""
        return (f"seed={self.seed} B={self.B} H={self.H}{kv} L={self.L} d={self.d} P={self.P} "
                f"causal={self.causal} layout={self.layout} dtype={self.dtype}")


def payloads(case: Case, names=("q", "k", "v")):
    return {n: syn.make_payload(case.seed, n, case.shape_of(n), case.dtype) for n in names}


def to_device(payload):
    import torch
    if payload.dtype == np.uint16:
        return torch.from_numpy(payload.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(payload).to("cuda")


def to_f64(t) -> np.ndarray:
    """Exact widening of a device tensor to a float64 numpy array."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rank_positions(case: Case, ranks):
    """Original token position of every local row of the given ranks: [nr, Bb]."""
    x = np.arange(case.Bb)
    return np.stack([oracle.token_position(case.layout, case.P, case.Bb, i, x) for i in ranks])


def lse_to_original(case: Case, lse_dev, ranks) -> tuple:
    """Device lse [nr, B, H, Bb] -> (positions [nr*Bb], values [B, nr*Bb, H])."""
    lse = lse_dev.cpu().numpy().astype(np.float64)  # [nr, B, H, Bb]
    pos = rank_positions(case, ranks).reshape(-1)
    vals = np.transpose(lse, (1, 0, 3, 2)).reshape(case.B, -1, case.H)
    return pos, vals


def bf16_half_spacing(x):
    """Half the distance between neighbouring bfloat16 numbers around |x|
    (8 significant bits): the most that rounding x to nearest bfloat16 moves
    it. |x| = m 2^e with 0.5 <= m < 1 gives spacing 2^(e-8)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    return np.where(ax > 0, np.ldexp(1.0, e - 9), 0.0)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def assert_close(name, got, ref, tol, case=None):
    err = max_abs(got, ref)
    scale = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    log(f"  {name}: max|err|={err:.3e} (tol {tol:g}, max|ref|={scale:.3g}) {case or ''}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values {case}"
    assert err <= tol, f"{name}: max abs error {err} > {tol} {case}"


def assert_output_close(name, got, ref, dtype, case=None):
    """An output returned in ``dtype``: max-abs error bar TOL[dtype] on the
    computed value, plus the output's own rounding when dtype is bfloat16."""
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype != "bf16" or not np.size(ref):
        assert_close(name, got, ref, tol, case)
        return
    err = np.abs(got - ref)
    # the value before rounding lies within tol of ref, and rounding moves it
    # by at most half the spacing at its magnitude
    beyond = float(np.max(err - bf16_half_spacing(np.maximum(np.abs(got), np.abs(ref) + tol))))
    log(f"  {name}: max|err|={float(np.max(err)):.3e}, beyond bf16 output rounding {beyond:.3e} "
        f"(tol {tol:g}, max|ref|={float(np.max(np.abs(ref))):.3g}) {case or ''}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values {case}"
    assert beyond <= tol, f"{name}: error beyond the bf16 output rounding {beyond} > {tol} {case}"
