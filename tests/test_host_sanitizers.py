"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every source with both sanitizers on its host code, links
tests/abi_sanitizer_driver.c against it and runs the driver with no GPU
visible: argument validation, size queries, workspace layouts and the grid
math of calls that pass validation (their launches then fail) run on the CPU
over fixed cases and 4000 rounds of random arguments for every entry point.
Any sanitizer report makes the driver exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

from video_dit_hybrid_amd import build as B

CLANG = "/opt/rocm/lib/llvm/bin/clang"
RT = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux"


@pytest.mark.skipif(not (os.path.exists(CLANG) and (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc"))),
                    reason="needs ROCm's hipcc and clang")
def test_abi_under_asan_and_ubsan(repo_root):
    lib = B.build_host_sanitized()
    libdir = os.path.dirname(lib)
    exe = os.path.join(libdir, "abi_driver")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-shared-libsan", "-I", os.path.join(repo_root, "include"),
                    os.path.join(repo_root, "tests", "abi_sanitizer_driver.c"), "-L", libdir,
                    "-lhybrid_attn_host_sanitized", "-L", "/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{libdir}",
                    f"-Wl,-rpath,{RT}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "all checks passed" in p.stdout
