"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the float64 oracle (oracle/gqa_oracle.c) and libgqa's planner and C ABI
checks (gqa_api.cpp, with the kernel launch stubbed out) are each built with
-fsanitize=address,undefined and driven over small shapes, edge cases and
bad arguments.  Any sanitizer report fails the run.  CPU only; built with
gcc / g++ (no GPU code is compiled here)."""
import os
import subprocess

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
HOST = os.path.join(ROOT, "tests", "host")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    r = _run(["gcc", "-std=gnu11", "-Wall", "-Wextra"] + SAN +
             [os.path.join(HOST, "oracle_check.c"), os.path.join(ROOT, "oracle", "gqa_oracle.c"),
              "-o", exe, "-lpthread", "-lm"])
    assert r.returncode == 0, r.stderr
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                             UBSAN_OPTIONS="print_stacktrace=1"), timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="needs the HIP runtime headers and library")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "planner_check")
    csrc = os.path.join(ROOT, "grouped_query_attention_decode_amd", "csrc")
    r = _run(["g++", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
              "-I", csrc, "-I", os.path.join(ROOT, "include")] + SAN +
             [os.path.join(HOST, "planner_check.cpp"), os.path.join(csrc, "gqa_api.cpp"),
              os.path.join(HOST, "kernel_stub.cpp"), "-o", exe,
              "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    assert r.returncode == 0, r.stderr
    # leaks inside the HIP runtime's own initialisation are not ours to find
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
                             HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", "")), timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
