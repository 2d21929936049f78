import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libbsa.so")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host time)")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_sparse_attention_plan_amd as bsa
    bsa.load_library()  # raises when the library is missing: no fallback
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Print the statistics of every full-size parity check that ran, so that
    they appear in the run's output even when test output is captured."""
    import parity_full
    if parity_full.REPORT:
        terminalreporter.section("full-size parity (every row / position against the oracle)")
        for line in parity_full.REPORT:
            terminalreporter.write_line(line)
