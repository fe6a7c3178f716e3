"""Build libsegkv.so (HIP kernels for gfx950 + host C++) in-tree.

    python head_segmented_paged_amd/build.py [--isa]

(Run it by path: importing the package loads the library being rebuilt.)

HIP sources go through hipcc for gfx950 only; host-only C++ goes through g++.
Every HIP compile carries `-Xclang -target-feature -Xclang -packed-fp32-ops`
(packed fp32 VALU ops are kept out of generated code).
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
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsegkv.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["segkv_attn.hip", "segkv_pages.hip", "segkv_ffn.hip"]
CXX_SOURCES = ["segkv_api.cpp", "segkv_tables.cpp"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    # the two-block prefill kernel's tile bodies are generated (no-op when current)
    _run([sys.executable, os.path.join(CSRC, "gen_tile_asm.py")])
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def isa(out_dir=BUILD):
    """Write the gfx950 assembly of the HIP sources (for register / occupancy review)."""
    os.makedirs(out_dir, exist_ok=True)
    for src in HIP_SOURCES:
        out = os.path.join(out_dir, src + ".s")
        _run([HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out])
    return out_dir


if __name__ == "__main__":
    build(verbose=True)
    if "--isa" in sys.argv:
        print(isa())
