"""Build libsmla.so in-tree with hipcc for gfx950.

Usage: python -m sparse_mla_attention_indices_amd.build [--verbose]
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsmla.so")
SOURCES = [os.path.join(CSRC, "smla_api.cpp"), os.path.join(CSRC, "smla_kernels.hip"),
           os.path.join(CSRC, "smla_attn128.hip")]
HEADERS = [os.path.join(ROOT, "include", "smla.h"), os.path.join(CSRC, "smla_internal.h"),
           os.path.join(CSRC, "smla_device.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU ops are disabled: the compiler must not emit them.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA results in ordinary registers (VGPR form): the two-wave-per-SIMD kernels
# then place operands in AGPRs without spilling, and attn128_kernel keeps its S^T
# accumulator there while O takes every AGPR through its written-out MFMA.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {"smla_kernels.hip": VGPR_FORM, "smla_attn128.hip": VGPR_FORM}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    """Compile every source (always, even if a library exists) and link libsmla.so."""
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *COMMON, "-x", "hip", "-c", src,
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
