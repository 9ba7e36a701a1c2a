import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """Write the near-margin counts the parity checkers gathered (per
    workload and decision kind) to the file DBV_PARITY_REPORT names."""
    path = os.environ.get("DBV_PARITY_REPORT")
    if not path:
        return
    try:
        from tests.parity import REPORT
    except Exception:  # pragma: no cover
        return
    if not REPORT:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as fh:
        json.dump({k: dict(v) for k, v in sorted(REPORT.items())}, fh, indent=1, sort_keys=True)
