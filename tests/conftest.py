import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionstart(session):
    # builds the library (hipcc for gfx950) when it is missing or was built from other
    # sources than the tree holds: the package refuses to import without it
    import runpy
    runpy.run_path(os.path.join(ROOT, "hashed_gram_memory_tid2eid_amd", "build_lib.py"))["ensure_built"]()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "pages_values.json")) as f:
        return json.load(f)
