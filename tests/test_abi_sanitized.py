"""The host side of the C ABI under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only).

Builds the library with every -fsanitize applied to the host pass only (the
device code is the same), then runs the host-side ABI tests in a child
process that preloads the AddressSanitizer runtime and loads that build.
Any sanitizer report makes the child fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    from linear_cross_entropy_02_amd import build as b
    try:
        b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = b.asan_runtime()
    if not rt or not os.path.exists(rt):
        pytest.skip("AddressSanitizer runtime not found")
    out = str(tmp_path_factory.mktemp("san") / "libflce_san.so")
    b.build(sanitize=True, out=out)
    return out, rt


def test_abi_under_address_and_ub_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import linear_cross_entropy_02_amd as f; f.load(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main([%r, '-q', '-p', 'no:cacheprovider']))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
