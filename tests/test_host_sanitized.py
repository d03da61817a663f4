"""The host cache manager under AddressSanitizer and UndefinedBehaviorSanitizer.

The host-logic suites (validation order, truncate/reset/fork bookkeeping,
block tables, ring caches, sessions) run again in a child process against a
build of kvc_host.cpp + tests/hostcheck_backend.cpp instrumented with
-fsanitize=address,undefined; any report fails the run.  The transactional
claims rest on this host code (Chapter 37, "Reset or reject without
corrupting retained state": a rejected call leaves the state unchanged).
CPU only: the instrumented code is host code built with g++.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_host_manager.py", "tests/test_host_paging.py", "tests/test_host_window.py",
          "tests/test_host_static_scratch.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_suites_are_clean_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    env = dict(os.environ)
    env["KVC_HOSTCHECK_FLAGS"] = ("-fsanitize=address,undefined -fno-sanitize-recover=all "
                                  "-fno-omit-frame-pointer")
    # the interpreter is not instrumented: the runtime must be loaded first, and
    # the interpreter's own allocations at exit are not this code's leaks
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *SUITES],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    report = "\n".join(l for l in r.stdout.splitlines()
                       if "Sanitizer" in l or "runtime error" in l or "passed" in l or "failed" in l)
    assert r.returncode == 0, r.stdout[-6000:]
    assert "runtime error" not in r.stdout and "ERROR: AddressSanitizer" not in r.stdout, report
    assert " passed" in r.stdout, r.stdout[-2000:]
