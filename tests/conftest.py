import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The sanitizer test (tests/test_sanitizers.py) runs the CPU tests again in
    # a child process against host-sanitized builds of the library and the
    # oracle, named by these variables.
    lib = os.environ.get("ATTN_TEST_LIB_PATH")
    if lib:
        import exact_attention_87_amd as ea

        ea.LIB_PATH = lib
    olib = os.environ.get("ATTN_TEST_ORACLE_LIB_PATH")
    if olib:
        import oracle

        oracle._LIB_PATH = olib


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build()
    return oracle
