"""Build libhybrid_attn.so (gfx950) in-tree with hipcc.

    python -m video_dit_hybrid_amd.build          # or __graft_entry__.build()

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU forms
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), then linked into
video_dit_hybrid_amd/libhybrid_attn.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libhybrid_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["hybrid_attn.hip", "attn_bf16.hip", "state_bf16.hip", "state_scan.hip", "fp32_path.hip", "fmap.hip",
           "gates.hip", "token_level.hip", "state_step.hip"]
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature flag; that warning is noise
    out = "\n".join(l for l in p.stdout.splitlines() if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


DEBUG_BUILD = os.path.join(BUILD, "debug")
DEBUG_LIB_PATH = os.path.join(PKG, "libhybrid_attn_debug.so")


def build(verbose: bool = False, extra_flags=(), debug: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path.
    debug: the same sources with -DHA_DEBUG (device index checks, reported by
    every entry point after synchronising its stream) into
    libhybrid_attn_debug.so beside the release library."""
    bdir, lib_path = (DEBUG_BUILD, DEBUG_LIB_PATH) if debug else (BUILD, LIB_PATH)
    extra_flags = (*extra_flags, "-DHA_DEBUG") if debug else tuple(extra_flags)
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIP_FLAGS, *extra_flags, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib_path)
    if verbose:
        print("built", lib_path)
    return lib_path


SANITIZE_DIR = os.path.join(BUILD, "host_sanitized")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "libhybrid_attn_host_sanitized.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on every host function
# (argument validation, workspace layout, grid math, launch order); the device
# code is built as usual and never sanitized. The driver that uses this library
# runs with no GPU visible, so its calls stop at failed launches.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host_sanitized(verbose: bool = False) -> str:
    """Every source with ASan + UBSan on its host code, linked into a shared
    library for the sanitizer driver (tests/abi_sanitizer_driver.c); returns its
    path. Without a visible GPU the library's launches fail cleanly (HA_ERR_DEVICE)."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(SANITIZE_DIR, src.replace(".hip", ".o"))
        cmd = [cc, f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", *SANITIZE_FLAGS,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd)
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", "-shared-libsan", *objs, "-o", SANITIZED_LIB])
    if verbose:
        print("built", SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        build_host_sanitized(verbose=True)
    else:
        build(verbose="-v" in sys.argv, debug="--debug" in sys.argv)
