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
