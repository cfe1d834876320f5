import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU sweeps")


def pytest_terminal_summary(terminalreporter):
    """Whole-tensor parity figures of the full-size workload comparisons that
    ran (their tests print them too, but a quiet run hides passing tests'
    output)."""
    parity = sys.modules.get("tests.parity")
    lines = getattr(parity, "SUMMARY", None)
    if lines:
        terminalreporter.section("whole-tensor parity against the oracle (every row)")
        for line in lines:
            terminalreporter.write_line(line)
