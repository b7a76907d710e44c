"""Build libprefill_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m rope_causal_attention_amd.build [--isa]``.  ``--isa`` also
writes the device assembly to ``_build/attn_kernels-gfx950.s`` for register
and scratch inspection.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libprefill_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.cpp", "rope_table.cpp", "attn_kernels.hip"]

# Packed fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose=False, isa=False):
    """Compile every source into LIB_PATH (always rebuilds)."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *DEVICE_FLAGS, *COMMON_FLAGS, "-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    if isa:
        bdir = os.path.join(ROOT, "_build")
        os.makedirs(bdir, exist_ok=True)
        asm = os.path.join(bdir, "attn_kernels-gfx950.s")
        cmd = [hipcc(), *DEVICE_FLAGS, *COMMON_FLAGS, "--cuda-device-only", "-S", "-o", asm,
               os.path.join(CSRC, "attn_kernels.hip")]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc -S failed:\n{res.stderr}")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, isa="--isa" in sys.argv[1:]))
