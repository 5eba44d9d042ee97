"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the library is rebuilt with host-side instrumentation (device code as
usual), and the C-ABI tests (validation of every entry point, workspace
sizing and carving, ternary quantisation and packing on the host) run
against it in a child Python with the sanitizer runtime preloaded.  Any
out-of-bounds access, use after free or undefined behaviour aborts the child.
The first run builds the library (about two minutes); later runs reuse it
until a source changes.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import sparse_activation_amd as qs
qs.load({lib!r})
import pytest
sys.exit(pytest.main([{tests!r}, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"]))
"""


def test_abi_under_asan_ubsan():
    from sparse_activation_amd import build
    try:
        runtime = build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_sanitized(verbose=False)
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
