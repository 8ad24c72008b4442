"""Sanitizer runs of the host code, on the CPU (not collected by pytest).

1. The oracle's C (oracle/gdn_oracle.c) built by gcc with AddressSanitizer
   and UndefinedBehaviorSanitizer, running tests/test_oracle.py against it.
2. libgdn.so built with host-side AddressSanitizer and
   UndefinedBehaviorSanitizer (hipcc: -Xarch_host before each sanitizer
   option, so no device code is instrumented), running tests/test_abi.py
   against it: argument validation, overlap and size checks, workspace
   sizes and exports.  Those calls return before any launch, so no GPU is
   needed, and the library's real host code is what runs.

Each run is a separate process with its own sanitizer runtime preloaded
(gcc's for the oracle, clang's for the HIP library); any report fails it.

Usage: python tests/sanitize.py
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "_build", "san")

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def runtime(compiler, name):
    return subprocess.run([compiler, f"-print-file-name={name}"], check=True, capture_output=True,
                          text=True).stdout.strip()


def run(tests, env_extra):
    env = dict(os.environ, **env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests]
    print("$", " ".join(f"{k}={v}" for k, v in env_extra.items()), " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


def main():
    os.makedirs(OUT, exist_ok=True)
    from oracle.build import build as build_oracle
    from linear_attention_recurrence_prep_amd.build import build as build_lib

    oracle_lib = build_oracle(verbose=True, lib=os.path.join(OUT, "libgdn_oracle_san.so"), extra_flags=GCC_SAN)
    gdn_lib = build_lib(verbose=True, extra_flags=HOST_SAN, lib=os.path.join(OUT, "libgdn_san.so"),
                        obj_dir=os.path.join(OUT, "obj"))
    rc = run(["tests/test_oracle.py"], {"LD_PRELOAD": runtime("gcc", "libasan.so"), "GDN_ORACLE_LIB": oracle_lib})
    if rc == 0:
        clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
        rc = run(["tests/test_abi.py"], {"LD_PRELOAD": runtime(clang, "libclang_rt.asan-x86_64.so"),
                                         "GDN_LIB": gdn_lib})
    print("sanitizer runs:", "clean" if rc == 0 else f"FAILED (exit {rc})", flush=True)
    return rc


if __name__ == "__main__":
    sys.exit(main())
