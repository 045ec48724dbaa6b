import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU oracle check")
    # CPU runs of the C-ABI tests against another build of the library (the
    # host-sanitizer build: python -m attention_delta_token_amd.build --host-asan)
    lib = os.environ.get("DASH_TEST_LIB")
    if lib:
        from attention_delta_token_amd import _lib
        _lib.load(lib)


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
