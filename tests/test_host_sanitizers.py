"""The host code of the C ABI under sanitizers, on the CPU: g++ builds of
zero_host.cpp and zero_offload.cpp with AddressSanitizer + UndefinedBehavior-
Sanitizer and with ThreadSanitizer run tests/host_sanitize_driver.cpp (the
planners, table preparation, argument checks of the device calls, the loss
scaler, and the offload form's host Adam with 1..16 worker threads at every
vector width, compared bit for bit with one scalar thread).  The device code
is never built with a sanitizer; no GPU is used."""
import os
import shutil
import subprocess

import pytest


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("kind", ["asan", "tsan"])
def test_host_code_is_clean_under_sanitizer(kind):
    from zero_sharded_optimizer_rank_amd import build

    res = build.build_host_sanitized(kind)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    r = subprocess.run([res["driver"]], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host sanitize driver: ok" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
