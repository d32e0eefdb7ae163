import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (minutes of CPU work)")


def pytest_sessionfinish(session, exitstatus):
    """Write the parity record (largest errors per compared configuration) when
    MLA_PARITY_REPORT names a file."""
    path = os.environ.get("MLA_PARITY_REPORT")
    if not path:
        return
    try:
        import parity
    except ImportError:
        return
    if not parity.RECORD:
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(parity.RECORD, f, indent=1, sort_keys=True)
