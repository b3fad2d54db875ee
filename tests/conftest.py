import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def ensure_library():
    """The built HIP library: tests load what is built and build it only when
    nothing is (a fresh checkout; about a minute of hipcc on the host)."""
    import route_dispatch_grouped_amd as rdg
    if not os.path.exists(rdg.LIB_PATH):
        from route_dispatch_grouped_amd.build import build
        build()
    return rdg.load_library()
