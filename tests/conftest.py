import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) and the built HIP library")


def _stale(lib, srcs):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="session")
def orc():
    import oracle

    src = os.path.join(ROOT, "oracle", "bitkv_oracle.c")
    hdr = os.path.join(ROOT, "oracle", "bitkv_oracle.h")
    oracle.build(force=_stale(oracle._LIB, [src, hdr]))
    return oracle
