import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


def pytest_sessionstart(session):
    """Build the HIP library when it is absent (hipcc cross-compiles without a
    GPU).  A present library is used as is: rebuild after changing a source."""
    from tiled_tensor_core_amd import attn, build

    if not os.path.exists(attn.LIB_PATH):
        build.build()
