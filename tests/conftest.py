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
    # the oracle is plain C built by gcc; build it once per session if absent
    from oracle import build as obuild
    if not os.path.exists(obuild.LIB):
        obuild.build()
    yield


def pytest_sessionfinish(session, exitstatus):
    # the parity checks' measured error margins, when asked for
    path = os.environ.get("PS_PARITY_MARGINS")
    if not path:
        return
    try:
        from tests import _harness
    except ImportError:
        return
    if _harness.MARGINS:
        import json
        with open(path, "w") as f:
            json.dump(_harness.MARGINS, f, indent=1)
