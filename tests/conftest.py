import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    """The CPU oracle (compiled with gcc if it is not built yet)."""
    import oracle
    if not os.path.exists(oracle.LIB):
        oracle.build()
    return oracle.Oracle()


def pytest_terminal_summary(terminalreporter):
    """The layer-output errors against the oracle of the parity cases that
    ran (printed even when test output is captured)."""
    try:
        from tests import gpu_helpers
    except Exception:  # noqa: BLE001 - no GPU helpers importable: nothing ran
        return
    if not gpu_helpers.RESULTS:
        return
    tr = terminalreporter
    tr.write_sep("-", "layer output vs the oracle (max_abs <= 2e-2, relL2 <= 5e-3)")
    for name, ma, rel, wr, nt in gpu_helpers.RESULTS:
        tr.write_line(f"{name}: max_abs={ma:.3e} relL2={rel:.3e} routing_w_rel={wr:.2e} "
                      f"near_ties={nt}")
