"""The library's host code under AddressSanitizer and UBSan (CPU only).

tests/asan_host_driver.cpp drives the C ABI in host-only mode (trees, plans,
views, growth, cost tables and every host-forced error path); it is built
here with g++ from the host sources, with both sanitizers on and any finding
fatal, and run.  No device code is involved: the kernel launchers are
stand-ins that fail if called."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_tree_amd", "csrc")
HOST = ["api.cpp", "host_tree.cpp", "host_plan.cpp", "cost_json.cpp"]


def test_host_code_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "asan_host_driver")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", os.path.join(ROOT, "tests", "asan_host_driver.cpp"),
           *[os.path.join(CSRC, s) for s in HOST], "-o", exe, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
           "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               PST_ASAN_TMP=str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "all checks passed" in r.stdout
