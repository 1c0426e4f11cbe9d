import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as O
    O.lib()
    return O


def pytest_terminal_summary(terminalreporter):
    """Every GPU-vs-oracle comparison of the session with its three error
    measures (also written to $CSA_PARITY_REPORT when set)."""
    try:
        from parity import REPORT
    except ImportError:
        return
    if not REPORT:
        return
    lines = [f"{'comparison':<70} {'normwise':>10} {'rms-scaled':>10} {'elementwise':>11}"]
    for what, nw, rw, el in REPORT:
        lines.append(f"{what[:70]:<70} {nw:10.3e} {rw:10.3e} {el:11.3e}")
    terminalreporter.write_sep("=", "parity report")
    for ln in lines:
        terminalreporter.write_line(ln)
    path = os.environ.get("CSA_PARITY_REPORT")
    if path:
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
