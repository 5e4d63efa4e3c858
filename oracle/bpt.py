"""A Blockwise Parallel Transformer layer in float64 — TEST INFRASTRUCTURE ONLY.

"Ring Attention 論文分析" (blog), section "BPT の Feedforward 融合": BPT
finishes each query block before it moves on. The block's attention output
goes through the output projection, a residual connection and layer
normalisation, then straight through the feedforward network, a second
residual connection and layer normalisation, and is written out. The
intermediate results of one block are never kept for the whole sequence,
which is what bounds the memory by the block size. The same section's layer
projects the whole sequence to Q, K and V first.

Written out here, per query block of ``block_size`` rows:
    y   = attn_out W_o^T + b_o              (attn_out: the heads side by side)
    h   = LN1(x_blk + y)
    f   = GELU(h W_1^T + b_1) W_2^T + b_2
    out = LN2(h + f)
with LN(z) = (z - mean(z)) / sqrt(var(z) + eps) * gamma + beta over the
model dimension (biased variance), and GELU the exact one,
0.5 z (1 + erf(z / sqrt(2))). Weights are stored [out, in], as the section's
linear layers hold them. Attention is the oracle's full-softmax definition
(oracle.attention), one head per d_model / n_heads columns.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from .attention import attention_fwd

LN_EPS = 1e-5  # the layer-normalisation default of the section's framework

PARAM_NAMES = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "ln1_g", "ln1_b",
               "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


def linear(x, w, b):
    """x [..., in] -> x W^T + b, W [out, in]."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T + np.asarray(b, np.float64)


def layer_norm(z, gamma, beta, eps=LN_EPS):
    z = np.asarray(z, np.float64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def gelu(z):
    z = np.asarray(z, np.float64)
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def ffn_block(attn_out, x_blk, p, round_to=None):
    """The block tail after attention: W_o, residual + LN1, FFN, residual + LN2.

    attn_out, x_blk: [rows, d_model]; p: dict of PARAM_NAMES arrays.
    Returns (out, h): the block output and the first normalised activations.
    ``round_to``, if given, is applied to the two activations the tail hands
    on as operands of its next products, h = LN1(...) and u = GELU(...):
    a device that keeps them in a narrower type rounds them there (tests use
    it to size the error that rounding alone causes); None keeps every value
    exact.
    """
    keep = round_to if round_to is not None else (lambda z: z)
    y = linear(attn_out, p["w_o"], p["b_o"])
    h = keep(layer_norm(np.asarray(x_blk, np.float64) + y, p["ln1_g"], p["ln1_b"]))
    u = keep(gelu(linear(h, p["w_1"], p["b_1"])))
    f = linear(u, p["w_2"], p["b_2"])
    return layer_norm(h + f, p["ln2_g"], p["ln2_b"]), h


def project_qkv(x, p, n_heads):
    """Q, K, V of the whole sequence as [B, L, H, d_k]."""
    B, L, dm = x.shape
    dk = dm // n_heads
    return tuple(linear(x, p[f"w_{n}"], p[f"b_{n}"]).reshape(B, L, n_heads, dk) for n in "qkv")


def bpt_layer(x, p, n_heads, block_size, causal=False, qkv=None):
    """The layer over x [B, L, d_model], one query block at a time.

    ``qkv`` may pass precomputed (Q, K, V) [B, L, H, d_k] (for instance the
    exact values a device computed) instead of projecting x.
    """
    x = np.asarray(x, np.float64)
    B, L, dm = x.shape
    if L % block_size:
        raise ValueError("the sequence must split into whole blocks")
    q, k, v = project_qkv(x, p, n_heads) if qkv is None else (np.asarray(t, np.float64) for t in qkv)
    out = np.zeros_like(x)
    for r0 in range(0, L, block_size):
        rows = np.arange(r0, r0 + block_size)
        o, _ = attention_fwd(q[:, rows], k, v, causal, q_pos=rows)
        for b in range(B):
            out[b, rows], _ = ffn_block(o[b].reshape(block_size, dm), x[b, rows], p)
    return out
