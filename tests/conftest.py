import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU case")


def read_golden(name):
    """Parse a golden fixture: '#' comments, whitespace-separated fields."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle
    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it runs (uncaptured), so that a
    run that dies inside a kernel still shows which case it was."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


@pytest.fixture(scope="session")
def bsfp():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_scaled_bit_fp_amd as b
    b.lib()
    return b
