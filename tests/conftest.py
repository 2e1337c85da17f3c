import os
import sys

import pytest

ROOT = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(ROOT)
for p in (REPO, ROOT):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # Use the library that is built; build it only when none is present.
    from long_context_block_amd import pisa

    if not os.path.exists(pisa.LIB_PATH):
        from long_context_block_amd import build

        build.build()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity counts and measured quantities of the GPU tests (units checked, decided fraction, errors,
    recall), printed even in a quiet run so that the record of the run keeps them."""
    mod = sys.modules.get("gpu_common")
    lines = getattr(mod, "SUMMARY", None) if mod else None
    if lines:
        terminalreporter.section("PISA parity summary")
        for line in lines:
            terminalreporter.write_line(line)
