"""Host-only checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, and of the library's logging and trace switches.

jl_rotated_bit_amd/build_hostsan.py builds the ABI layer and the host table
generators with both sanitizers and links tests/native/hostsan_driver.cpp
against them; the driver calls every host generator and every entry point
with arguments that validation must reject (no call reaches the GPU).  CPU
only.
"""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "jl_rotated_bit_amd", "csrc", f)
           for f in ("qjl_abi.hip", "sketch.cpp", "rotq_host.cpp", "internal.h", "qjl_testing.h")]
SOURCES += [os.path.join(ROOT, "include", "qjl.h"), os.path.join(ROOT, "tests", "native", "hostsan_driver.cpp"),
            os.path.join(ROOT, "jl_rotated_bit_amd", "build_hostsan.py")]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


@pytest.fixture(scope="module")
def driver():
    from jl_rotated_bit_amd import build_hostsan
    path = build_hostsan.DRIVER
    newest = max(os.path.getmtime(s) for s in SOURCES)
    if not os.path.exists(path) or os.path.getmtime(path) < newest:
        path = build_hostsan.build()
    return path


def run(driver, **env):
    e = dict(os.environ)
    for k in ("QJL_LOG", "QJL_TRACE"):
        e.pop(k, None)
    e.update(SAN_ENV)
    e.update(env)
    return subprocess.run([driver], capture_output=True, text=True, env=e, timeout=300)


def test_abi_clean_under_address_and_ub_sanitizers(driver):
    r = run(driver)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert "[qjl]" not in r.stderr          # silent unless QJL_LOG is set


def test_qjl_log_reports_errors_and_calls(driver):
    r = run(driver, QJL_LOG="1")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "[qjl] error 2: qjl_encode_keys: " in r.stderr      # an unsupported shape
    assert "[qjl] qjl_encode_keys\n" not in r.stderr           # calls only at level 2
    r = run(driver, QJL_LOG="2")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "[qjl] qjl_encode_keys\n" in r.stderr
    assert "[qjl] qjl_tq_scores\n" in r.stderr


def test_qjl_trace_ranges_load_roctx(driver):
    """QJL_TRACE=1 opens roctx ranges around every call (no profiler needed:
    the ranges are then no-ops); the calls behave exactly as without it."""
    r = run(driver, QJL_TRACE="1", QJL_LOG="1")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all checks passed" in r.stdout
    assert "no roctx library found" not in r.stderr
