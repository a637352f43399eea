"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host translation unit (argument validation, workspace layouts,
the balance statistics' host group array, the timing bookkeeping) is rebuilt
with both sanitizers on its host code only and linked, ahead of the normal
libmoe.so (which supplies the kernel launchers), into a small driver that
calls every entry point with arguments its validation rejects.  No HIP call
is reached, so no GPU is needed; a sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_ffn_fp32_amd")
LIB = os.path.join(PKG, "libmoe.so")
ROCM = "/opt/rocm"


def _tool(path):
    if not os.path.exists(path):
        pytest.skip(f"{path} not available")
    return path


def test_abi_host_code_is_sanitizer_clean(tmp_path):
    hipcc = _tool(os.path.join(ROCM, "bin", "hipcc"))
    clang = _tool(os.path.join(ROCM, "llvm", "bin", "clang++"))
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built: run python -m mixture_experts_ffn_fp32_amd.build")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = tmp_path / "moe_api_san.o"
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                        "-c", os.path.join(PKG, "csrc", "moe_api.hip"), "-o", str(api_o)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_host_checks"
    r = subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "sanitize", "abi_host_checks.cpp"),
                        str(api_o), LIB, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", f"-Wl,-rpath,{PKG}",
                        "-o", str(exe)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "ALL OK" in r.stdout, out[-4000:]
