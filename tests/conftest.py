import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case")


# Lines that parity tests want in the run's own log (tie counts, measured
# errors): printed in the terminal summary, so they appear with -q and with
# output capture on.
REPORT_LINES = []


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if REPORT_LINES:
        terminalreporter.section("parity measurements")
        for line in REPORT_LINES:
            terminalreporter.write_line(line)


def read_golden(name):
    """Non-comment, non-empty lines of a golden fixture."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.rstrip("\n") for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library on a machine with a GPU; fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_11_amd import _lib
    return _lib.load()
