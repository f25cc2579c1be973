import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def dv():
    """The HIP-backed package; GPU tests fail loudly if the library is not built."""
    import contextual_activation_sparsity_amd as pkg
    pkg.require_gpu()
    return pkg


def pytest_terminal_summary(terminalreporter):
    """How many chained set comparisons differed from the oracle's own top-k, and by how much
    (printed when any GPU test compared sets)."""
    try:
        from helpers import ERRORS, SET_DRIFT
    except ImportError:
        return
    if ERRORS:
        by_bar = {}
        for what, ratio, bar in ERRORS:
            if ratio > by_bar.get(bar, ("", -1.0))[1]:
                by_bar[bar] = (what, ratio)
        for bar in sorted(by_bar):
            what, ratio = by_bar[bar]
            terminalreporter.write_line(f"largest layer error held to the internal bar {bar:g} x RMS: "
                                        f"{ratio:.2e} x RMS ({what})")
    if not SET_DRIFT:
        return
    rows = len(SET_DRIFT)
    differ = [r for r in SET_DRIFT if r[3] > 0]
    worst = max(SET_DRIFT, key=lambda r: r[3])
    terminalreporter.write_line(
        f"selected-set drift: {rows} rows compared with the oracle's own top-k, {len(differ)} differ at near ties; "
        f"largest difference {worst[3]} indices ({worst[0]}, row {worst[1]}, k {worst[2]}, "
        f"{worst[4]} oracle scores inside the tie band)")
