import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU for inputs)")


def pytest_sessionstart(session):
    # the host sanitizer test reruns the host modules against a sanitized
    # build of the library's host code, named by PA_TEST_LIB
    path = os.environ.get("PA_TEST_LIB")
    if path:
        from paged_kv_cache_443_amd import _lib

        _lib.LIB_PATH = path
        print(f"pa library: {path}", flush=True)
