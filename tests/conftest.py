import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # Use the library that is built; build it only when none is present.
    from long_context_block_amd import pisa

    if not os.path.exists(pisa.LIB_PATH):
        from long_context_block_amd import build

        build.build()
