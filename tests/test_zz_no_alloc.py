"""ra_backward_noalloc, the backward for callers that cannot allocate: the
library's static scratch (D and lse in base-2 units) replaces the workspace.
Checked through the C ABI against ra_backward on the same inputs and
against the float64 oracle at the parity bar, on two calls in a row, the
second on a smaller problem, so that the scratch holds the first call's rows
when the second starts. dK and dV come from the same kernel in both and
must agree bit for bit; ra_backward with its full workspace takes dQ from
the stored dS, the no-allocation call recomputes it, so dQ agrees to the
bar (fp32 sums in another order)."""
import numpy as np
import pytest

import exact_blockwise_attention_amd as ra
import oracle
from gpu_cases import Case, assert_output_close, log, payloads, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    Case(191, 2, 4, 2048, 128, 4, True, "striped", "bf16"),
    Case(192, 1, 2, 600, 64, 3, True, "contiguous", "bf16", Hk=1),  # smaller, after the first
]


def test_noalloc_backward_matches_the_workspace_backward():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ra.library()
    for case in CASES:
        log(f"no-allocation backward {case}")
        p = payloads(case, ("q", "k", "v", "do"))
        dev = {n: to_device(x) for n, x in p.items()}
        o, lse = ra.attention_forward(dev["q"], dev["k"], dev["v"], case.P, case.layout, case.causal)
        ref = ra.attention_backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.P, case.layout,
                                    case.causal)
        got = ra.attention_backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.P, case.layout,
                                    case.causal, noalloc=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dK", "dV"), got[1:], ref[1:]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from ra_backward"
        assert_output_close("dQ vs ra_backward", to_f64(got[0]), to_f64(ref[0]), case.dtype, case)
        f = {n: oracle_input(x) for n, x in p.items()}
        dq_r, dk_r, dv_r, _, _ = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], case.causal)
        for name, a, r in zip(("dQ", "dK", "dV"), got, (dq_r, dk_r, dv_r)):
            assert_output_close(name, to_f64(a), r, case.dtype, case)


def test_noalloc_backward_rejects_a_problem_beyond_its_scratch():
    """Checked before anything is enqueued: no GPU work runs."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = Case(193, 1, 32, 8 * 65536, 128, 8, True, "striped", "bf16")  # 128 MiB of rows: over 64 MiB
    pb = ra.make_problem(case.B, case.H, case.d, case.P, case.Bb, case.layout, True, ra.BF16)
    assert ra.workspace_bytes(pb, 0, case.P, False, 2) > ra.backward_noalloc_max_bytes()
    s = ra.Seq(0x10000, 128, 1 << 20, 4096, 128)
    with pytest.raises(ra.RaError) as e:
        ra.backward_noalloc_raw(pb, 0, case.P, s, s, s, s, s, 0x20000, s, s, s, ra._stream_handle(None))
    assert e.value.status == 7


def oracle_input(x):
    from exact_blockwise_attention_amd import synthetic as syn
    return syn.to_f64(x)
