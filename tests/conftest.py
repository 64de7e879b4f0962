import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to a minute)")


def pytest_report_header(config):
    return f"few_row_vocab tests, root {ROOT}"


@pytest.fixture(autouse=True)
def _announce(request):
    # Name every test before it starts, so a run that dies mid-test still says which one.
    print(f"\n[start] {request.node.nodeid}", flush=True)
    yield


def pytest_terminal_summary(terminalreporter):
    mod = sys.modules.get("tests.parity") or sys.modules.get("parity")
    if mod is not None and mod.WORST["what"]:
        terminalreporter.write_line(
            f"largest logit error relative to its tolerance: {mod.WORST['ratio']:.3e} "
            f"({mod.WORST['what']})")
