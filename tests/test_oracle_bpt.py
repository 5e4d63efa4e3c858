"""Pins of the float64 BPT-layer oracle (oracle/bpt.py) against facts that do
not come from it: torch's CPU float64 linear, layer-norm, GELU and attention
routines assembled as the blog's layer; the method's own identity (the output
does not depend on the block size); textbook GELU values; closed forms of
layer normalisation; and planted mistakes that must fail a pin."""
import math

import numpy as np
import pytest

import oracle.bpt as ob

torch = pytest.importorskip("torch")


def params(seed, dm, dff):
    """Linear weights [out, in] uniform in +-1/sqrt(in), biases and the
    normalisation's gamma/beta near (1, 0)."""
    rng = np.random.default_rng(seed)
    p = {}
    for n, (o, i) in {"q": (dm, dm), "k": (dm, dm), "v": (dm, dm), "o": (dm, dm),
                      "1": (dff, dm), "2": (dm, dff)}.items():
        p[f"w_{n}"] = rng.uniform(-1, 1, (o, i)) / math.sqrt(i)
        p[f"b_{n}"] = rng.uniform(-1, 1, o) / math.sqrt(i)
    for n in ("ln1", "ln2"):
        p[f"{n}_g"] = 1.0 + 0.1 * rng.standard_normal(dm)
        p[f"{n}_b"] = 0.1 * rng.standard_normal(dm)
    return p


def torch_layer(x, p, n_heads, causal):
    """The blog's layer with torch's own routines, over the whole sequence."""
    t = {k: torch.tensor(v) for k, v in p.items()}
    X = torch.tensor(x)
    B, L, dm = X.shape
    F = torch.nn.functional
    heads = lambda z: z.reshape(B, L, n_heads, dm // n_heads).transpose(1, 2)  # noqa: E731
    q, k, v = (heads(F.linear(X, t[f"w_{n}"], t[f"b_{n}"])) for n in "qkv")
    a = F.scaled_dot_product_attention(q, k, v, is_causal=causal).transpose(1, 2).reshape(B, L, dm)
    normed = F.layer_norm(X + F.linear(a, t["w_o"], t["b_o"]), (dm,), t["ln1_g"], t["ln1_b"], eps=1e-5)
    f = F.linear(F.gelu(F.linear(normed, t["w_1"], t["b_1"])), t["w_2"], t["b_2"])
    return F.layer_norm(normed + f, (dm,), t["ln2_g"], t["ln2_b"], eps=1e-5).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_layer_matches_torch_f64(causal):
    B, L, dm, H, dff = 2, 24, 16, 4, 40
    x = np.random.default_rng(1).standard_normal((B, L, dm))
    p = params(2, dm, dff)
    out = ob.bpt_layer(x, p, H, block_size=8, causal=causal)
    assert np.max(np.abs(out - torch_layer(x, p, H, causal))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_output_does_not_depend_on_the_block_size(causal):
    """The BPT identity: finishing one query block at a time gives the
    layer's output over the whole sequence, for every block size."""
    B, L, dm, H, dff = 1, 48, 16, 2, 32
    x = np.random.default_rng(3).standard_normal((B, L, dm))
    p = params(4, dm, dff)
    ref = ob.bpt_layer(x, p, H, block_size=L, causal=causal)
    for bs in (24, 12, 8, 1):
        assert np.max(np.abs(ob.bpt_layer(x, p, H, block_size=bs, causal=causal) - ref)) < 1e-13


def test_gelu_textbook_values():
    # GELU(z) = z Phi(z), Phi the standard normal distribution function
    phi1 = 0.8413447460685429  # Phi(1)
    g = ob.gelu(np.array([0.0, 1.0, -1.0, 8.0, -8.0]))
    assert g[0] == 0.0
    assert abs(g[1] - phi1) < 1e-15
    assert abs(g[2] + (1.0 - phi1)) < 1e-15
    assert abs(g[3] - 8.0) < 1e-12 and abs(g[4]) < 1e-12


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((7, 33)) * 3 + 2
    y = ob.layer_norm(z, np.ones(33), np.zeros(33), eps=0.0)
    assert np.max(np.abs(y.mean(axis=-1))) < 1e-14
    assert np.max(np.abs((y ** 2).mean(axis=-1) - 1.0)) < 1e-13
    beta = rng.standard_normal(33)
    const = np.full((3, 33), 4.5)
    assert np.max(np.abs(ob.layer_norm(const, rng.standard_normal(33), beta) - beta)) < 1e-15


def test_planted_tanh_gelu_is_caught(monkeypatch):
    """The tanh approximation of GELU in the oracle fails the torch pin."""
    B, L, dm, H, dff = 1, 16, 16, 2, 32
    x = np.random.default_rng(6).standard_normal((B, L, dm)) * 3
    p = params(7, dm, dff)
    ref = torch_layer(x, p, H, False)
    monkeypatch.setattr(ob, "gelu", lambda z: 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3))))
    assert np.max(np.abs(ob.bpt_layer(x, p, H, block_size=8) - ref)) > 1e-6


def test_planted_unbiased_variance_is_caught(monkeypatch):
    B, L, dm, H, dff = 1, 16, 16, 2, 32
    x = np.random.default_rng(8).standard_normal((B, L, dm))
    p = params(9, dm, dff)
    ref = torch_layer(x, p, H, True)

    def ln_unbiased(z, gamma, beta, eps=ob.LN_EPS):
        mu = z.mean(axis=-1, keepdims=True)
        var = ((z - mu) ** 2).sum(axis=-1, keepdims=True) / (z.shape[-1] - 1)
        return (z - mu) / np.sqrt(var + eps) * gamma + beta

    monkeypatch.setattr(ob, "layer_norm", ln_unbiased)
    assert np.max(np.abs(ob.bpt_layer(x, p, H, block_size=8, causal=True) - ref)) > 1e-3


def test_rounded_intermediates_are_h_and_the_gelu_output():
    """ffn_block's round_to reaches exactly the two activations the tail
    hands on to its next products, LN1's output and GELU's output (checked
    against torch's routines), and changes nothing when it is the identity;
    rounding them changes the output through both the FFN and the second
    residual (torch with the same roundings agrees)."""
    rng = np.random.default_rng(9)
    rows, dm, dff = 5, 16, 40
    p = params(10, dm, dff)
    a, x = rng.standard_normal((rows, dm)), rng.standard_normal((rows, dm))
    seen = []
    out_id, h_id = ob.ffn_block(a, x, p, round_to=lambda z: seen.append(z.copy()) or z)
    out, h = ob.ffn_block(a, x, p)
    assert np.array_equal(out_id, out) and np.array_equal(h_id, h)
    t = {k: torch.tensor(v) for k, v in p.items()}
    F = torch.nn.functional
    normed = F.layer_norm(torch.tensor(x) + F.linear(torch.tensor(a), t["w_o"], t["b_o"]), (dm,), t["ln1_g"],
                          t["ln1_b"], eps=1e-5)
    u = F.gelu(F.linear(normed, t["w_1"], t["b_1"]))
    assert len(seen) == 2
    assert np.max(np.abs(seen[0] - normed.numpy())) < 1e-12
    assert np.max(np.abs(seen[1] - u.numpy())) < 1e-12
    coarse = lambda z: np.round(z * 8) / 8  # noqa: E731
    out_c, _ = ob.ffn_block(a, x, p, round_to=coarse)
    nc = torch.tensor(coarse(normed.numpy()))
    uc = torch.tensor(coarse(F.gelu(F.linear(nc, t["w_1"], t["b_1"])).numpy()))
    want = F.layer_norm(nc + F.linear(uc, t["w_2"], t["b_2"]), (dm,), t["ln2_g"], t["ln2_b"], eps=1e-5).numpy()
    assert np.max(np.abs(out_c - want)) < 1e-12
    assert np.max(np.abs(out_c - out)) > 1e-3
