import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large oracle work (seconds to a minute on the host)")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; fail loudly rather than skip when they are selected
    # explicitly on a machine that has one but lacks the library (that is handled in the tests).
    pass
