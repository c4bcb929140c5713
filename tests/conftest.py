import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Print the full-size parity results (max-abs and relative Frobenius error
    against the fp64 oracle) that the GPU tests recorded."""
    mod = sys.modules.get("gpu_util")
    rows = getattr(mod, "PARITY_REPORT", None) if mod else None
    if not rows:
        return
    terminalreporter.write_sep("-", "parity vs fp64 oracle (full-size workloads)")
    for what, max_abs, rel in rows:
        terminalreporter.write_line(f"{what:<44} max-abs {max_abs:.3e}  rel-fro {rel:.3e}")
