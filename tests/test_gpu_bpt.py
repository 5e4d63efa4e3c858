"""GPU parity of the Blockwise Parallel Transformer layer around attention
(ra_linear, ra_layer_norm, ra_bpt_ffn and the composed layer) against the
float64 oracle (oracle/bpt.py), on exactly the bf16/fp32 values the GPU sees.

Bars: fp32 outputs of a product of bf16 operands accumulated in fp32 within
1e-4 (max abs, N(0, 1)-scale values); bf16 outputs within 2e-2 beyond their
own rounding to bfloat16 (tests/gpu_cases.py assert_output_close). The layer
tail keeps h = LN1(...) and u = GELU(...) in bfloat16 as the operands of its
next products; the error that rounding alone causes (the oracle run exact and
with those two values rounded) is allowed on top of the bar. Small cases
use ragged row counts (not a multiple of the 256-row tile or of the block);
the full-size layer tail is checked on a spread of rows, each of which the
oracle computes on its own (every row of the tail is independent).
"""
import numpy as np
import pytest

import exact_blockwise_attention_amd as ra
import oracle.bpt as ob
from exact_blockwise_attention_amd import synthetic as syn
from gpu_cases import assert_close, assert_output_close, log, round_bf16, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.library()


def dev_params(p):
    return {k: to_device(v) for k, v in p.items()}


def f64_params(p):
    return {k: syn.to_f64(v) for k, v in p.items()}


def ffn_reference(attn, x, p):
    """The oracle's tail, exact, and the error its bf16 intermediates h and
    u cause on their own."""
    a, xx, pp = syn.to_f64(attn), syn.to_f64(x), f64_params(p)
    ref, _ = ob.ffn_block(a, xx, pp)
    ref_bf16, _ = ob.ffn_block(a, xx, pp, round_to=round_bf16)
    return ref, np.abs(ref_bf16 - ref)


@pytest.mark.parametrize("m,n,k,bias,res,gelu,f32", [
    (300, 256, 192, True, False, False, True),
    (300, 256, 192, True, True, False, True),
    (300, 384, 256, True, False, True, False),
    (512, 128, 64, False, True, True, False),
    (7, 128, 128, True, True, True, True),
])
def test_linear_epilogues(m, n, k, bias, res, gelu, f32):
    log(f"linear m={m} n={n} k={k} bias={bias} res={res} gelu={gelu} f32={f32}")
    seed = 400 + m + n + k
    a = syn.make_payload(seed, "x", (m, k), "bf16")
    w = syn.f32_to_bf16_bits(syn.normal_f32(seed, "w_1", (n, k)) / np.float32(np.sqrt(k)))
    b = syn.normal_f32(seed, "b_1", (n,))
    r = syn.make_payload(seed, "attn", (m, n), "bf16")
    out = ra.linear(to_device(a), to_device(w), to_device(b) if bias else None, to_device(r) if res else None,
                    gelu=gelu, out_f32=f32)
    torch.cuda.synchronize()
    ref = ob.linear(syn.to_f64(a), syn.to_f64(w), b if bias else np.zeros(n))
    if res:
        ref = ref + syn.to_f64(r)
    if gelu:
        ref = ob.gelu(ref)
    if f32:
        assert_close("linear fp32", to_f64(out), ref, 1e-4)
    else:
        assert_output_close("linear bf16", to_f64(out), ref, "bf16")


@pytest.mark.parametrize("rows,d", [(37, 384), (256, 4096), (3, 8192)])
def test_layer_norm(rows, d):
    log(f"layer norm rows={rows} d={d}")
    z = syn.normal_f32(500 + d, "x", (rows, d)) * np.float32(3.0) + np.float32(1.5)
    g = syn.normal_f32(500 + d, "ln1_g", (d,))
    b = syn.normal_f32(500 + d, "ln1_b", (d,))
    out = ra.layer_norm(to_device(z), to_device(g), to_device(b))
    torch.cuda.synchronize()
    assert_output_close("layer norm", to_f64(out), ob.layer_norm(z.astype(np.float64), g, b), "bf16")


@pytest.mark.parametrize("rows,dm,dff,block", [(600, 256, 512, 256), (512, 384, 1024, 512), (130, 128, 256, 64)])
def test_bpt_ffn_small(rows, dm, dff, block):
    """The layer tail, block by block, with a ragged last block."""
    seed = 600 + rows
    log(f"bpt ffn rows={rows} d_model={dm} d_ff={dff} block={block}")
    attn = syn.make_payload(seed, "attn", (rows, dm), "bf16")
    x = syn.make_payload(seed, "x", (rows, dm), "bf16")
    p = syn.bpt_params(seed, dm, dff)
    out = ra.bpt_ffn(to_device(attn), to_device(x), dev_params(p), block)
    torch.cuda.synchronize()
    ref, allow = ffn_reference(attn, x, p)
    assert_output_close("bpt ffn", to_f64(out), ref, "bf16", allowance=allow)


@pytest.mark.parametrize("causal", [False, True])
def test_bpt_layer_small(causal):
    """Projections, ring attention and the tail, composed from library calls,
    against the oracle's layer (its own Q, K, V from x)."""
    B, L, dm, H, dff, P = 1, 512, 256, 2, 512, 4
    seed = 700 + int(causal)
    log(f"bpt layer L={L} d_model={dm} heads={H} d_ff={dff} P={P} causal={causal}")
    x = syn.make_payload(seed, "x", (B, L, dm), "bf16")
    p = syn.bpt_params(seed, dm, dff)
    out = ra.bpt_layer(to_device(x), dev_params(p), H, P, block_rows=128, causal=causal)
    torch.cuda.synchronize()
    ref = ob.bpt_layer(syn.to_f64(x), f64_params(p), H, block_size=L // P, causal=causal)
    assert_output_close("bpt layer", to_f64(out), ref, "bf16")


def test_bpt_ffn_full_size_sampled_rows():
    """The 7B-shaped tail (d_model 4096, d_ff 16384, 4096-row blocks) over
    32768 rows; the oracle recomputes a spread of rows."""
    w = syn.BPT_WORKLOAD
    log(f"bpt ffn full size {w['name']}")
    rows, dm, dff = w["rows"], w["d_model"], w["d_ff"]
    attn = syn.make_payload(w["wid"], "attn", (rows, dm), "bf16")
    x = syn.make_payload(w["wid"], "x", (rows, dm), "bf16")
    p = syn.bpt_params(w["wid"], dm, dff)
    out = ra.bpt_ffn(to_device(attn), to_device(x), dev_params(p), w["block_rows"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(71)
    sel = np.unique(np.concatenate([[0, rows - 1, w["block_rows"] - 1, w["block_rows"]],
                                    rng.choice(rows, 60, replace=False)]))
    ref, allow = ffn_reference(attn[sel], x[sel], p)
    got = to_f64(out[torch.as_tensor(sel, device="cuda")])
    assert_output_close("bpt ffn full size", got, ref, "bf16", w["name"], allowance=allow)
