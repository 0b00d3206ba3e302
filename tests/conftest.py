import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """After a GPU session: the per-tensor parity errors of every comparison against the oracle."""
    gu = sys.modules.get("tests.gpu_util")
    if gu is None or not getattr(gu, "RECORDS", None):
        return
    table = gu.parity_table()
    terminalreporter.write_sep("-", "parity errors against the oracle (rel = max|gpu-ref| / max|ref|)")
    terminalreporter.write_line(table)
    path = os.environ.get("SARATHI_PARITY_TABLE")
    if path:
        with open(path, "w") as f:
            f.write(table + "\n")
