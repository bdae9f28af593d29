"""CPU sanitizer run: the oracle and the C-ABI host code under AddressSanitizer
and UndefinedBehaviorSanitizer.

    python tests/sanitize_cpu.py

Builds, under _build/sanitize/ (not committed):
  * the oracle (oracle/smla_oracle.c) with gcc -fsanitize=address,undefined;
  * libsmla.so with its host code (csrc/smla_api.cpp: argument validation, the
    split planner, the workspace contract, the prefill chunk planner) compiled
    by hipcc with AddressSanitizer and UndefinedBehaviorSanitizer on the host
    side only, and the unchanged GPU kernel objects;
then runs, each in its own process with the matching sanitizer runtime
preloaded (gcc's for the oracle, clang's for the library; one runtime per
process):
  * tests/test_oracle_pins.py and tests/test_oracle_mutants.py against the
    sanitized oracle (SMLA_ORACLE_LIB);
  * tests/test_abi.py (exports, validation, plans, no-ops; no GPU calls)
    against the sanitized library (SMLA_LIB_PATH).
Any sanitizer report stops the process (halt_on_error) and fails the run.
Leak detection is off: the Python interpreter itself does not free
everything at exit. Exit status 0 means every run passed.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
PKG = os.path.join(ROOT, "sparse_mla_attention_indices_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, env=env, cwd=ROOT)
    if r.returncode != 0:
        sys.exit(f"failed ({r.returncode}): {' '.join(cmd)}")


def build_oracle() -> str:
    lib = os.path.join(OUT, "libsmla_oracle.so")
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-fopenmp",
         os.path.join(ROOT, "oracle", "smla_oracle.c"), "-o", lib, "-lm"])
    return lib


def build_library() -> str:
    api_o = os.path.join(OUT, "smla_api.o")
    kern_os = [os.path.join(OUT, "smla_kernels.o"), os.path.join(OUT, "smla_attn128.o")]
    lib = os.path.join(OUT, "libsmla.so")
    dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]
    run([HIPCC, *dev, *common, *host_san, "-x", "hip", "-c",
         os.path.join(PKG, "csrc", "smla_api.cpp"), "-o", api_o])
    for src, obj in zip(("smla_kernels.hip", "smla_attn128.hip"), kern_os):
        run([HIPCC, *dev, "-O3", "-std=c++17", "-fPIC", "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-I",
             os.path.join(ROOT, "include"), "-x", "hip", "-c", os.path.join(PKG, "csrc", src), "-o", obj])
    # host-only link with clang++ (the kernel objects carry their own device code)
    run([CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", api_o, *kern_os,
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    return lib


def main() -> None:
    os.makedirs(OUT, exist_ok=True)
    oracle_lib = build_oracle()
    smla_lib = build_library()
    gcc_rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
              for n in ("libasan.so", "libubsan.so")]
    clang_rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        sys.exit("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm")
    pytest = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=":".join(gcc_rt), SMLA_ORACLE_LIB=oracle_lib)
    run([*pytest, "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"], env=env)
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=clang_rt[-1], SMLA_LIB_PATH=smla_lib)
    run([*pytest, "tests/test_abi.py"], env=env)
    print("sanitizer runs passed", flush=True)


if __name__ == "__main__":
    main()
