"""Build ``libgdn.so`` (gfx950 kernels + C ABI) in-tree with hipcc.

Usage: ``python -m linear_attention_recurrence_prep_amd.build`` (or call
``build()``).  Objects go to ``_build/``; the library is written next to
this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")

SOURCES = ["gdn_api.cpp", "prep.hip", "recurrent.hip", "chunked.hip", "epilogue.hip", "scratch.hip"]
# Matrix-core accumulators in ordinary VGPRs (no AGPR copies around the
# element-wise work on them).
SOURCE_FLAGS = {"chunked.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
# Packed FP32 instructions are disabled for every HIP translation unit: the
# compiler then emits only scalar v_fma_f32 / v_mul_f32 / v_add_f32 forms.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None, lib=LIB, obj_dir=OUT_DIR, link_flags=None) -> str:
    """Compile every source and link ``lib`` (default: the in-tree
    libgdn.so).  extra_flags / link_flags are appended to the compile and
    link lines (a sanitizer build passes host-only flags and another path)."""
    os.makedirs(obj_dir, exist_ok=True)
    extra = list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; drop that note
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l or "error" in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), flush=True)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *(link_flags or []), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


C_DEMO_SRC = os.path.join(ROOT, "tests", "c_abi_demo.c")
C_DEMO = os.path.join(ROOT, "tests", "c_abi_demo")


def build_c_abi_demo(verbose: bool = False) -> str:
    """Compile the C99 test program of the ABI (tests/c_abi_demo.c) with gcc
    against the in-tree libgdn.so and the HIP runtime (no HIP device code)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = C_DEMO + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), C_DEMO_SRC,
           "-L", PKG, "-lgdn", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../linear_attention_recurrence_prep_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, C_DEMO)
    return C_DEMO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    build_c_abi_demo(verbose="-v" in sys.argv)
    print(LIB)
