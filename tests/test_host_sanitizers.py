"""Host code under AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer (CPU only, g++):

* the C ABI's host side -- plan.cpp (schedule, workspace layout) and
  capi.cpp (validation, stage loops, chunk tables, stream and event
  ordering, timing) -- linked against host stand-ins of the kernel
  launchers and HIP runtime calls (tests/sanitize/hip_stubs.cpp), driven by
  tests/sanitize/host_driver.cpp;
* the fp64 oracle, every entry point, driven by tests/sanitize/oracle_driver.cpp.

Any sanitizer report aborts the program (-fno-sanitize-recover), so the test
fails on the first one.  No GPU code is built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "headwise_chunked_context_stage_amd", "csrc")
FLAGS = ["-std=c++17", "-g", "-O1", "-pthread", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_and_run(tmp_path, name, sources, extra):
    exe = str(tmp_path / name)
    res = subprocess.run(["g++"] + FLAGS + extra + sources + ["-o", exe], capture_output=True,
                         text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(run.stdout[-2000:])
    assert run.returncode == 0, (run.stdout[-4000:], run.stderr[-4000:])
    assert "ok:" in run.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_c_abi_host_code_under_sanitizers(tmp_path):
    build_and_run(tmp_path, "host_asan",
                  [os.path.join(SAN, "host_driver.cpp"), os.path.join(SAN, "hip_stubs.cpp"),
                   os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "capi.cpp")],
                  ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"])


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_sanitizers(tmp_path):
    build_and_run(tmp_path, "oracle_asan",
                  [os.path.join(SAN, "oracle_driver.cpp"), os.path.join(ROOT, "oracle", "upipe_oracle.cpp")],
                  ["-ffp-contract=off"])
