"""The C ABI layer (api.cpp and the host planning in plan.cpp) built for the
host alone under AddressSanitizer and UndefinedBehaviorSanitizer, with the
kernel launchers replaced by stubs (tests/sanitize/stub_launchers.cpp), and
driven through every entry point: valid shapes of every size class (the
largest workloads included) reach the launch dispatch, and every invalid
argument returns its status before anything is launched
(tests/sanitize/abi_driver.cpp).  No GPU: the stubs never touch the fake
device pointers.  Any sanitizer report aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_block_sparse_dsa_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")]
    # host code only: each sanitizer flag is scoped to the host compilation
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, f"driver failed ({run.returncode}):\n{run.stdout}\n{run.stderr}"
    assert "abi driver ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
