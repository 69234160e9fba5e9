import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def kda_lib():
    """The HIP library for host-only tests, built in-tree if it is missing
    (GPU runs load the library built beforehand and never build)."""
    import kda_chunked_delta_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        from kda_chunked_delta_amd import build as kbuild
        kbuild.build(verbose=False)
    return kda.lib()
