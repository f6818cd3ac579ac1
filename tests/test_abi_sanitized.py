"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): a copy of the library built with both on its host code runs the
ABI tests (symbol exports, argument checks and their error codes, workspace
queries, the measurement hook's arguments) in a child process that preloads
the sanitizer runtime; any report ends that process with an error."""
import os
import subprocess
import sys

import pytest

from draft_verify_sampling_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    try:
        build.build(sanitize=True)
        return build.sanitizer_env(os.environ)
    except RuntimeError as e:  # no hipcc or no sanitizer runtime in this image
        pytest.skip(f"sanitized build unavailable: {e}")


def test_abi_tests_pass_under_sanitizers(san_env):
    # the child loads the sanitized copy, with the runtime in its address space
    probe = ("import draft_verify_sampling_amd as sv; sv.load(); "
             "maps = open('/proc/self/maps').read(); "
             "assert sv.lib_path().endswith('_build/san/libspecverify.so'), sv.lib_path(); "
             "assert 'libclang_rt.asan' in maps and '_build/san/libspecverify.so' in maps; print('loaded')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=san_env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=san_env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr
