import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    _oracle.build(force=False)
    return _oracle


def pytest_sessionfinish(session, exitstatus):
    # the parity statistics of every element-wise check (max error over the
    # tolerance, max relative error, normwise error), for the record
    path = os.environ.get("SSM_PARITY_STATS")
    if not path:
        return
    from tests._parity import RECORD

    if RECORD:
        import json

        with open(path, "w") as f:
            json.dump(RECORD, f, indent=0)
