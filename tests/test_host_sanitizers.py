"""The host layer of the C ABI (argument validation, the planner counts, the resume records,
the thread-local error text) built from its source with the address and undefined-behaviour
sanitizers, and separately with the thread sanitizer, and run on the CPU: the kernel launchers
are replaced by stand-ins that report "no device" (tests/host/launch_stubs.cpp), so every call
runs its whole host path. No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "ring_sequence_parallelism_ra_amd", "csrc")


def compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no clang++")


@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_abi_host_layer_under_sanitizers(tmp_path, san):
    exe = str(tmp_path / "abi_checks")
    cmd = [compiler(), "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={san}",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "ra_api.cpp"),
           os.path.join(HOST, "launch_stubs.cpp"), os.path.join(HOST, "abi_checks.cpp"), "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and ("unsupported" in r.stderr or "cannot find" in r.stderr):
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "all passed" in run.stdout
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr[-4000:]
