import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name):
    """Parse a ``tests/golden`` fixture: ``name v1 v2 ...`` lines, ``#`` comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


@pytest.fixture(scope="session")
def golden():
    return load_golden


def pytest_terminal_summary(terminalreporter):
    """Per-layer ReLU-mask counts of the GPU parity checks: every row of the
    named workloads, and one aggregate line for the other cases."""
    try:
        from tests import parity
        from mlp_gemm_softmax_amd import synth
    except Exception:
        return
    rows = parity.MASK_REPORT
    if not rows:
        return
    tr = terminalreporter
    tr.section("ReLU mask bits (GPU against the float64 oracle and against its own operands)")
    tr.write_line("case | layer | units | oracle band | adopted | outside | self band | self differ in | self differ out")
    named = [r for r in rows if r[0].split()[-1] in synth.WORKLOADS]
    for r in named:
        tr.write_line(" | ".join("-" if v is None else str(v) for v in r))
    other = [r for r in rows if r[0].split()[-1] not in synth.WORKLOADS]
    if other:
        worst = max(other, key=lambda r: r[4] / r[2])
        tr.write_line(f"other cases: {len(other)} layer checks, adopted at most {worst[4] / worst[2]:.2e} "
                      f"of a layer's units ({worst[0]} layer {worst[1]}), "
                      f"{sum(r[5] for r in other)} bits outside the oracle's band")
