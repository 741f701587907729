"""The host scheduler (cpa_sched.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer, under the host-scheduler tests: no memory error
and no undefined behaviour while every descriptor still matches the oracle.
CPU only (g++)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_scheduler_suite_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("no sanitizer runtimes")
    lib = tmp_path / "libcpa_sched_sanitized.so"
    build = subprocess.run(
        ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared", "-fPIC",
         "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "chunked_prefill_paged_amd", "csrc", "cpa_sched.cpp"), "-o", str(lib)],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_under_sanitizer.py"), str(lib)],
                         capture_output=True, text=True, env=env, timeout=600)
    log = run.stdout + run.stderr
    assert run.returncode == 0, log[-4000:]
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert " passed" in log
