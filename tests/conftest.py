import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# A build of the library other than the in-tree libfa.so (a sanitized host build, or a variant
# under measurement) can be put under every test by naming it in FA_TEST_LIBRARY.
if os.environ.get("FA_TEST_LIBRARY"):
    import io_aware_exact_23_amd as _fa

    _fa._LIB_PATH = os.path.abspath(os.environ["FA_TEST_LIBRARY"])
