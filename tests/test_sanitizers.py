"""The host block pool (paged_kv_cache_255_amd/csrc/pool.cpp) and the CPU
oracle (oracle/pa_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and driven by seeded random operation streams
(tests/sanitize/).  Both drivers also check invariants that hold whatever the
placement policy: reference counts against the exported tables for the pool,
finite outputs, refused bad inputs and the one-token closed form for the
oracle.  A sanitizer report aborts the driver, which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, exe):
    subprocess.check_call(cmd)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pool_ops")
    csrc = os.path.join(ROOT, "paged_kv_cache_255_amd", "csrc")
    out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
                os.path.join(ROOT, "tests", "sanitize", "pool_ops.cpp"),
                os.path.join(csrc, "pool.cpp"), os.path.join(csrc, "errors.cpp"), "-o", exe],
               exe)
    assert "0 failed checks" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_ops")
    out = _run(["gcc", "-std=gnu11", *SAN, os.path.join(ROOT, "tests", "sanitize", "oracle_ops.c"),
                "-o", exe, "-lm", "-lpthread"], exe)
    assert "0 failed checks" in out
