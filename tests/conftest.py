import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Prints what the parity tests compared (pairs, worst errors) even under -q, where
    the tests' own output is captured."""
    here = os.path.dirname(os.path.abspath(__file__))
    if here not in sys.path:
        sys.path.insert(0, here)
    mod = sys.modules.get("kda_testlib")
    lines = getattr(mod, "REPORT", []) if mod else []
    if lines:
        terminalreporter.section("parity checked against the oracle")
        for ln in lines:
            terminalreporter.write_line(ln)
