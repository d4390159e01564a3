"""The C ABI's host code under the address and undefined-behaviour sanitizers: gdn_api.cpp is
rebuilt with them (the kernels' objects from the last build are linked as they are) and
tests/test_abi.py runs against that library in a child process with the sanitizer runtime
preloaded. A sanitizer report aborts the child, which fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    from linear_attention_recurrence_amd import build as b
    if not os.path.exists(b.SANITIZER_RUNTIME):
        pytest.skip("no sanitizer runtime at %s" % b.SANITIZER_RUNTIME)
    if not all(os.path.exists(os.path.join(b.BUILD_DIR, s + ".o")) for s in b.SOURCES if s.endswith(".hip")):
        pytest.fail("the kernels are not built; run __graft_entry__.build()")
    lib = b.build_host_sanitized()
    env = dict(os.environ)
    env.update(GDN_LIBRARY=lib, LD_PRELOAD=b.SANITIZER_RUNTIME,
               # Python's own allocations are not this library's; every error aborts
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
