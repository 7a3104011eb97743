"""The C-ABI validation layer under host-side sanitizers.

api.hip's host code (argument checks, workspace carving, error strings) is
rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer and the CPU ABI
tests (tests/test_abi.py: every invalid configuration, size query and
validation-only call, no GPU work) run against it in a child interpreter with
the sanitizer runtime preloaded.  Any report fails the test.
"""
import os
import subprocess
import sys

import pytest

from bit_attention_video_amd import build as vbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    rt = vbuild.asan_runtime()
    if rt is None or not os.path.exists(vbuild.hipcc()):
        pytest.skip("no hipcc or AddressSanitizer runtime")
    try:
        lib = vbuild.build_sanitized(str(tmp_path))
    except FileNotFoundError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "VCATTN_LIBRARY": lib,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
