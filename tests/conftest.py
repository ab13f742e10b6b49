import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libdg.so")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Every parity error the GPU tests measured, against its gate."""
    try:
        from helpers import PARITY_RECORDS
    except ImportError:  # pragma: no cover
        return
    if not PARITY_RECORDS:
        return
    tr = terminalreporter
    tr.section("parity: measured error / gate")
    for test, what, err, gate in PARITY_RECORDS:
        tr.write_line(f"{err:10.3e} / {gate:8.1e}  {test}  {what}")
