"""The planner and the C-ABI's host paths built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU (no GPU, no device code).

`tests/host/plan_checks.cpp` drives the host-only descriptor builders over
random multi-segment sequences, suffix queries and key chunks (empty ones,
also on the last sequence), the pages' workload shapes and the 2^31
head-span limit, checks the planner's invariants against the mask's
definition, replays every K/V tile load range of every work item with the
range functions the kernels use, and checks that invalid arguments come back
as status codes. Any sanitizer report or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_varlen_masked_attn_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compiler():
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ and the HIP headers are needed for the host sanitizer build")
    return gxx


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("host_san") / "plan_checks")
    cmd = [_compiler(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "host", "plan_checks.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "api.cpp"), "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"sanitizer build failed:\n{res.stderr[-4000:]}"
    return exe


def test_planner_and_abi_under_sanitizers(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([checker, "400"], capture_output=True, text=True, timeout=600, env=env)
    print(res.stdout)
    assert res.returncode == 0, f"host checks failed (exit {res.returncode}):\n{res.stdout}\n{res.stderr[-6000:]}"
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-6000:]
