"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU tests of its argument checks and of the
binding's checks run in a child process against a build of libwq whose host
code carries both sanitizers (loaded through WQ_LIBRARY, with the ASan
runtime preloaded); any report fails the test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from bit_quantized_linear_int4_amd import _build  # noqa: E402


def _have_hipcc():
    try:
        _build.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_abi_checks_clean_under_asan_and_ubsan():
    lib = _build.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "WQ_LIBRARY": lib,
        "LD_PRELOAD": _build.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(ROOT, "tests", "test_abi.py"),
         os.path.join(ROOT, "tests", "test_binding_checks.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
