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

    @property
    def Bb(self):
        return self.L // self.P

    @property
    def shape(self):
        return (self.B, self.L, self.H, self.d)

    def __str__(self):
        return (f"seed={self.seed} B={self.B} H={self.H} L={self.L} d={self.d} P={self.P} "
                f"causal={self.causal} layout={self.layout} dtype={self.dtype}")


def payloads(case: Case, names=("q", "k", "v")):
    return {n: syn.make_payload(case.seed, n, case.shape, case.dtype) for n in names}


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


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def assert_close(name, got, ref, tol, case=None):
    err = max_abs(got, ref)
    scale = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    log(f"  {name}: max|err|={err:.3e} (tol {tol:g}, max|ref|={scale:.3g}) {case or ''}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values {case}"
    assert err <= tol, f"{name}: max abs error {err} > {tol} {case}"
