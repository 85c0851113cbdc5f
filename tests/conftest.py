import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _sanitized_blocks_library():
    """Under tests/test_sanitizers.py the allocator batteries run against a host-only build of
    the block allocator with ASan/UBSan (PKV_TEST_BLOCKS_LIB); the binding's loader is
    pointed at it here, in the test process only."""
    path = os.environ.get("PKV_TEST_BLOCKS_LIB")
    if not path:
        return
    import ctypes

    from paged_kv_cache_80_amd import blocks

    lib = ctypes.CDLL(path)
    lib.pkv_last_error.restype = ctypes.c_char_p
    blocks.load = lambda: lib


_sanitized_blocks_library()


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built once per session from oracle/pkv_oracle.c; under
    tests/test_sanitizers.py the sanitized build named by PKV_TEST_ORACLE_LIB)."""
    import oracle

    path = os.environ.get("PKV_TEST_ORACLE_LIB")
    if path:
        oracle._lib = oracle.load(path)  # every oracle call of this process uses it
        return oracle
    oracle.build()
    oracle.load()
    return oracle
