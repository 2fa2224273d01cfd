import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are only meaningful where a GPU is visible; on a CPU-only host they are
    # deselected by -m "not gpu".  If they are selected without a GPU, fail loudly
    # rather than silently skipping the native path.
    pass
