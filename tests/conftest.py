import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    # The oracle is test infrastructure; build it with gcc if it is not there yet.
    from oracle import oracle as O
    if not os.path.exists(O.LIB):
        O.build_oracle()
    yield


def pytest_sessionfinish(session, exitstatus):
    """Write the parity class counts of the run to $DDT_PARITY_JSON, if set."""
    path = os.environ.get("DDT_PARITY_JSON")
    if not path:
        return
    try:
        from parity_util import RECORD
    except ImportError:
        return
    if not RECORD:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exit_status": int(exitstatus), "counts": RECORD}, f, indent=1, sort_keys=True)
