"""Build libvrcomm.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m collective_window_put_amd.build        # or build() from Python

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into collective_window_put_amd/libvrcomm.so. Flags: gfx950 only; packed fp32
instructions disabled in device code; IEEE fp32 denormals kept; no fast-math.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvrcomm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link; returns the library path. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


NATIVE = os.path.join(ROOT, "tests", "native")


def build_c_client(verbose: bool = False) -> str:
    """Compile tests/native/allreduce_worked_example.c, a plain C client of the
    library (gcc, C11, the HIP runtime's C API), next to its source; it finds
    libvrcomm.so through a path relative to itself. Returns the binary's path."""
    src = os.path.join(NATIVE, "allreduce_worked_example.c")
    out = os.path.join(NATIVE, "allreduce_worked_example")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(rocm, "include"), "-I" + os.path.join(ROOT, "include"), src,
           "-L" + PKG, "-lvrcomm", "-L" + os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../collective_window_put_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {src}:\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_c_client(verbose=True)
