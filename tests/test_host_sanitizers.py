"""The library's host-only code (csrc/dah_host.cpp: argument validation, the
split planner, status strings, the per-thread last error) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer and driven through its
rejection paths, planner grid and error buffer (tests/native/
host_checks_driver.cpp).  Any out-of-bounds access, overflow or leak the
sanitizers see aborts the driver; any status other than the expected one is
a failure line."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_head_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "native", "host_checks_driver.cpp")
HOST = os.path.join(CSRC, "dah_host.cpp")


def _build(tmp_path, flags):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_checks")
    cmd = [gxx, "-std=c++17", "-g", "-fno-omit-frame-pointer", *flags, f"-I{INCLUDE}",
           f"-I{CSRC}", DRIVER, HOST, "-o", exe, "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in " ".join(flags) and "asan" in res.stderr.lower():
        pytest.skip("sanitizer runtime not available: " + res.stderr[-300:])
    assert res.returncode == 0, res.stderr
    return exe


def _run(exe):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    last = res.stdout.strip().splitlines()[-1]
    checks, failures = int(last.split()[1]), int(last.split()[3])
    assert failures == 0 and checks > 500, last
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr


def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    _run(_build(tmp_path, ["-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]))


def test_host_code_optimised_build(tmp_path):
    _run(_build(tmp_path, ["-O3"]))
