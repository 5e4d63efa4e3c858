import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter):
    """The raw max-abs errors of every output the GPU parity tests compared
    (gpu_cases.RECORDS), one line per output, so that they are part of the
    run's record even under -q."""
    mod = sys.modules.get("gpu_cases")
    recs = getattr(mod, "RECORDS", None) if mod else None
    recs = [r for r in (recs or []) if "test_gpu" in r[0]]
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity: raw max |GPU - oracle| per compared output")
    tr.write_line("test | output | raw max|err| | max|err| at |ref|<4 | elements |ref|>=4 | max|err| there | max|ref|")
    worst = {}
    for test, name, raw, below, n_band, in_band, scale in recs:
        tr.write_line(f"{test} | {name} | {raw:.3e} | {below:.3e} | {n_band} | {in_band:.3e} | {scale:.3g}")
        key = name.split("[")[0].split(" ")[0]
        w = worst.setdefault(key, [0.0, 0.0, 0, 0.0])
        w[0] = max(w[0], raw)
        w[1] = max(w[1], below)
        w[2] += n_band
        w[3] = max(w[3], in_band)
    tr.write_line("worst per output: " + "; ".join(
        f"{k} raw {v[0]:.3e}, below 4 {v[1]:.3e}, {v[2]} at >=4 (max {v[3]:.3e})" for k, v in sorted(worst.items())))
