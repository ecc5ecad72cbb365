"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with the host code instrumented (device code as in the
product), then tests/test_abi_host.py -- every validation path, the workspace
queries, the shape limits -- runs in a child process that preloads the ASan
runtime and loads that build.  Any out-of-bounds access, use after free or
undefined behaviour (signed overflow, bad shift, misaligned access) in the host
code aborts the child.  No GPU is touched: every call there fails validation
or the device check before a launch.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    from nvfp4_w4a4_mixture_amd import build

    try:
        lib = build.build(sanitize=True)
        rt = build.asan_runtime()
    except RuntimeError as e:  # pragma: no cover - toolchain without the runtime
        pytest.skip(str(e))
    return lib, rt


def _env(lib, rt):
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, MOE_NVFP4_LIB=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_sanitized_build_is_instrumented_and_loaded(sanitized):
    lib, rt = sanitized
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle_" in syms
    code = "from nvfp4_w4a4_mixture_amd import _lib; print(_lib.lib()._name)"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == lib


def test_abi_validation_under_sanitizers(sanitized):
    lib, rt = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=_env(lib, rt), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
