"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of the library with both sanitizers on its host pass only
(device code is built as usual) and a C driver, tests/c_abi/gqa_host_checks.c,
with the same sanitizers; the driver walks the host-side argument checks of
every entry point and the pure-host split-count and workspace rules. A
sanitizer report, or any unexpected status, fails the test. CPU only: no call
reaches the GPU. Builds into pytest's temporary directory (about 30 s).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_checks_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    inc, csrc = os.path.join(ROOT, "include"), os.path.join(ROOT, "decode_attention_gqa_amd", "csrc")
    lib = str(tmp_path / "libgqa_decode.so")
    exe = str(tmp_path / "gqa_host_checks")
    build_lib = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-I", inc, "-I", csrc, os.path.join(csrc, "gqa_decode.hip"), "-o", lib]
    build_driver = [clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", inc,
                    os.path.join(ROOT, "tests", "c_abi", "gqa_host_checks.c"),
                    "-L", str(tmp_path), "-lgqa_decode", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    for cmd in (build_lib, build_driver):
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout + r.stderr)
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.returncode == 0
    assert "host checks: 0 failure(s)" in r.stdout
