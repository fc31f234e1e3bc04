"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
host-only sanitized build of the library (no kernels registered) runs every test of
test_abi_cpu.py (argument checks, aliasing, workspace and size queries at extreme sizes,
the Python bindings' validation) in a child process with the clang ASan runtime preloaded.
Any sanitizer report aborts the child and fails this test."""
import glob
import os
import subprocess
import sys

import pytest

from dynamic_short_convolution_amd import build

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib: str) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(build.CSRC, "*")) + glob.glob(os.path.join(REPO, "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        runtime = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(f"no sanitizer runtime: {e}")
    lib = build.ASAN_LIB_PATH
    if _stale(lib):
        build.build_host_sanitized()
    return lib, runtime


def test_abi_under_asan_and_ubsan(sanitized_lib):
    lib, runtime = sanitized_lib
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, DYNCONV_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(REPO, "tests", "test_abi_cpu.py"), "-x", "-q", "-s",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    res = subprocess.run(cmd, cwd=REPO, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in out


def test_sanitized_library_is_the_one_loaded(sanitized_lib):
    """The child really runs the sanitized build: its exports match and it is instrumented."""
    lib, runtime = sanitized_lib
    env = dict(os.environ, LD_PRELOAD=runtime, DYNCONV_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0")
    code = ("from dynamic_short_convolution_amd import _lib; l = _lib.load(); "
            "import ctypes; print(l._name); print(bool(ctypes.CDLL(None).__asan_init))")
    res = subprocess.run([sys.executable, "-c", code], cwd=REPO, env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = res.stdout.split()
    assert lines[0] == lib and lines[1] == "True"
