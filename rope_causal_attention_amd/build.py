"""Build libprefill_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m rope_causal_attention_amd.build [--isa]``.  Each source is
compiled to an object under ``_build/`` (in parallel), then linked.  ``--isa``
also writes the device assembly of each ``.hip`` source to
``_build/<name>-gfx950.s`` for register and scratch inspection.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libprefill_attn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.cpp", "rope_table.cpp", "attn_kernels.hip", "decode_kernels.hip", "device_peak.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")

# Packed fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, isa=False):
    """Compile every source and link LIB_PATH (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc(), *DEVICE_FLAGS, *COMMON_FLAGS, "-c", "-o", obj, os.path.join(CSRC, src)])
        if isa and src.endswith(".hip"):
            asm = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + "-gfx950.s")
            jobs.append([hipcc(), *DEVICE_FLAGS, *COMMON_FLAGS, "--cuda-device-only", "-S", "-o", asm,
                         os.path.join(CSRC, src)])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), *DEVICE_FLAGS, "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, isa="--isa" in sys.argv[1:]))
