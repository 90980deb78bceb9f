"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C entry points, the argument validation and the block manager are plain
C++ (the kernels live in separate HIP sources).  They are compiled here with
g++ -fsanitize=address,undefined into a host-only library whose kernel
launchers report "no device" (tests/sanitize/launch_stubs.cpp), and the host
test modules -- every rejection case of the C ABI and the block manager's
4000 random operations against the oracle's -- run again in a child process
that loads that library instead of the HIP build.  Any sanitizer report
fails the child (halt_on_error), so the test fails.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_443_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("pa_api.cpp", "pa_validate.cpp", "pa_block_manager.cpp")]
STUBS = os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")
MODULES = ["tests/test_abi_host.py", "tests/test_block_manager_host.py"]


def _runtime(name: str):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if shutil.which("g++") is None or _runtime("libasan.so") is None:
        pytest.skip("g++ with libasan is not available")
    out = tmp_path_factory.mktemp("asan")
    lib = str(out / "libpa_host_asan.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           *HOST_SOURCES, STUBS, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib


def test_host_code_is_clean_under_asan_and_ubsan(sanitized_lib):
    env = dict(os.environ)
    env.update({
        "PA_TEST_LIB": sanitized_lib,
        "LD_PRELOAD": _runtime("libasan.so"),
        # the interpreter itself is not instrumented: leaks at its exit are not ours
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *MODULES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-6000:]
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-6000:]
    # the child really loaded the sanitized library (conftest prints it)
    assert f"pa library: {sanitized_lib}" in text, text[-3000:]
