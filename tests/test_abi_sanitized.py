"""The host ABI tests again, against a build whose C ABI layer carries
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; see
tests/sanitize_build.py).  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_tests_under_sanitizers(tmp_path):
    from tests import sanitize_build

    try:
        lib = sanitize_build.build(str(tmp_path))
    except RuntimeError as e:
        pytest.fail(str(e))
    env = dict(os.environ)
    env.update(LD_PRELOAD=sanitize_build.runtime(), SHERRY_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
