"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer: the validation tests of test_abi.py run against
a host-only build of api.cpp and the planning code (kernel launchers
stubbed), in a child process with the sanitizer runtimes preloaded; any
sanitizer report aborts it."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(name):
    return subprocess.check_output(["g++", f"-print-file-name={name}"], text=True).strip()


def test_abi_validation_under_asan_and_ubsan():
    from linear_attention_lm_amd.build import build_sanitized

    lib = build_sanitized()
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("sanitizer runtimes not installed")
    env = dict(os.environ, BASED_LIB_PATH=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", "not every_declared_symbol and not product_path"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log
    assert " passed" in r.stdout, log
