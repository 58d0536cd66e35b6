"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on the
CPU: the C ABI's validation and routing (kda_api.cpp, with the kernel launchers
replaced by recording stand-ins, tests/sanitize/launch_stubs.cpp) and the fp64
oracle (oracle/kda_ref.c). Each is built with gcc/g++ into a temporary
directory and run by a small driver; any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
SAN_FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_api_host_code_under_sanitizers(tmp_path):
    need("g++")
    if not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("HIP headers not installed")
    exe = str(tmp_path / "api_driver")
    cmd = ["g++", "-std=c++17", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "gated_delta_rule_63_amd", "csrc", "kda_api.cpp"),
           os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "api_driver.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe]
    rc, out = run(cmd)
    assert rc == 0, out
    # HIP_VISIBLE_DEVICES="" keeps the driver off any GPU: only host code runs
    rc, out = run([exe], env=dict(ENV, HIP_VISIBLE_DEVICES=""), timeout=120)
    assert rc == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "all expectations met" in out


def test_oracle_under_sanitizers(tmp_path):
    need("gcc")
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c11", *SAN_FLAGS, os.path.join(ROOT, "oracle", "kda_ref.c"),
           os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe]
    rc, out = run(cmd)
    assert rc == 0, out
    rc, out = run([exe], env=ENV, timeout=120)
    assert rc == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "all checks passed" in out
