import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

# The library compiles kernels for programs without an ahead-of-time kernel in
# a background thread by default, switching launches from the interpreter to
# the compiled kernel whenever the compile ends.  Tests pin the kernel each
# launch uses: run-time compilation is off unless a test turns it on (the
# background mode has tests of its own).
os.environ.setdefault("ECMD_JIT", "0")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only sweep")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle
    oracle.build()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stdout before it touches the GPU."""
    if request.node.get_closest_marker("gpu") is not None:
        print("\n[gpu-case] %s" % request.node.nodeid, flush=True)
    yield
