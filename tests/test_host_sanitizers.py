"""The host layer (la_gdn_api.cpp: argument checks, workspace carving, stride
normalisation, options, profiler) built for the CPU under AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers and the HIP runtime
replaced by stand-ins (tests/host_sanitize/hip_stubs.cpp), and driven through
the C ABI by tests/host_sanitize/abi_driver.cpp.  No GPU and no device code:
the kernels are not part of this build."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ (host compiler with the sanitizer runtimes) absent")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    # host-only C++ (no offload): the sanitizers apply to the CPU code alone
    cmd = [CLANG, "-x", "c++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gated_delta_rule_50_amd", "csrc"), "-I" + HERE,
           os.path.join(ROOT, "gated_delta_rule_50_amd", "csrc", "la_gdn_api.cpp"),
           os.path.join(HERE, "hip_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
