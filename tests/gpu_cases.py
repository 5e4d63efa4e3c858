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

# Max-abs error bars against the float64 oracle: 2e-2 for bf16 inputs with
# fp32 accumulation, 1e-4 for fp32 inputs. Every element of O, dQ, dK and dV
# whose exact value is below BAND in magnitude must meet the plain bar, which
# already absorbs the output's own rounding to bfloat16 there (half a bf16
# spacing is at most 2^-7 below 4). Only at |ref| >= BAND, where rounding to
# bfloat16 alone moves a value by up to 2^-6 (0.031 from 8 on), does a bf16
# output get that half spacing on top of the bar. lse is fp32 and always gets
# the plain bar.
TOL = {"bf16": 2e-2, "f32": 1e-4}
BAND = 4.0

# One record per compared output: (test id, output name, raw max |err|, max
# |err| below BAND, elements at or above BAND, max |err| there, max |ref|).
# conftest.py prints them at the end of the run, so that the raw errors show
# even under `pytest -q`.
RECORDS = []


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


def lse_at_tokens(layout, P, Bb, lse_dev, tokens, heads) -> np.ndarray:
    """Device lse [P, B, H, Bb] (all ranks, local row order) at the given
    original token positions and heads: [B, len(tokens), len(heads)]."""
    lse = lse_dev.cpu().numpy().astype(np.float64)
    pos_all = np.concatenate([oracle.token_position(layout, P, Bb, i, np.arange(Bb)) for i in range(P)])
    where = np.empty_like(pos_all)
    where[pos_all] = np.arange(pos_all.size)  # token -> rank-major local index
    idx = where[np.asarray(tokens)]
    ri, x = idx // Bb, idx % Bb
    return np.stack([lse[ri, :, h, x] for h in heads], axis=-1).transpose(1, 0, 2)


def bf16_half_spacing(x):
    """Half the distance between neighbouring bfloat16 numbers around |x|
    (8 significant bits): the most that rounding x to nearest bfloat16 moves
    it. |x| = m 2^e with 0.5 <= m < 1 gives spacing 2^(e-8)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)
    return np.where(ax > 0, np.ldexp(1.0, e - 9), 0.0)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def _current_test():
    import os
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]


def assert_close(name, got, ref, tol, case=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = max_abs(got, ref)
    scale = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    RECORDS.append((_current_test(), name, err, err, 0, 0.0, scale))
    msg = f"{name}: max|err|={err:.3e} (tol {tol:g}, max|ref|={scale:.3g}) {case or ''}"
    log("  " + msg)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values {case}"
    assert err <= tol, msg


def round_bf16(x):
    """x rounded to the nearest bfloat16 (through float32, as a device
    rounds its fp32 values), widened back to float64."""
    x = np.asarray(x, dtype=np.float64)
    return syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def assert_output_close(name, got, ref, dtype, case=None, allowance=None):
    """An output returned in ``dtype``. The plain bar TOL[dtype] on every
    element with |ref| < BAND (and on all of them for fp32); at |ref| >=
    BAND a bfloat16 output may in addition be off by the half bf16 spacing
    that rounding it to the output type costs at that magnitude.
    ``allowance`` (per element, default 0) is subtracted from the error
    first: the error that intermediate values kept in bfloat16 cause on
    their own, where a computation prescribes them (sized by the caller
    with the oracle)."""
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype != "bf16" or not np.size(ref):
        assert allowance is None
        assert_close(name, got, ref, tol, case)
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values {case}"
    err = np.abs(got - ref)
    if allowance is not None:
        raw_err = float(np.max(err))
        err = np.maximum(err - np.asarray(allowance, dtype=np.float64), 0.0)
        log(f"  {name}: raw max|err| {raw_err:.3e}, allowance for bf16 intermediates up to "
            f"{float(np.max(allowance)):.3e}")
    band = np.abs(ref) >= BAND
    raw = float(np.max(err))
    below = float(np.max(err[~band])) if np.any(~band) else 0.0
    n_band = int(np.count_nonzero(band))
    in_band = float(np.max(err[band])) if n_band else 0.0
    # in the band: the value before rounding lies within tol of ref, and
    # rounding moves it by at most half the spacing at its magnitude
    beyond = 0.0
    if n_band:
        mag = np.maximum(np.abs(got[band]), np.abs(ref[band]) + tol)
        beyond = float(np.max(err[band] - bf16_half_spacing(mag)))
    scale = float(np.max(np.abs(ref)))
    RECORDS.append((_current_test(), name, raw, below, n_band, in_band, scale))
    msg = (f"{name}: max|err|={raw:.3e}; |ref|<{BAND:g}: {below:.3e} (tol {tol:g}); "
           f"|ref|>={BAND:g}: {n_band} elements, max|err| {in_band:.3e}, beyond output rounding "
           f"{beyond:.3e}; max|ref|={scale:.3g} {case or ''}")
    log("  " + msg)
    assert below <= tol, msg
    assert beyond <= tol, msg
