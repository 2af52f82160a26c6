"""Build libqbl.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libqbl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qbl_gemv.hip", "qbl_batched.hip", "qbl_jit.hip", "qbl_dar.hip", "qbl_probe.hip", "qbl_static.hip",
           "qbl_format.cpp", "qbl_runtime.cpp"]
# Packed fp32 VALU ops are disabled on purpose (the flag only affects device code).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


# Per-source flags.  qbl_gemv.hip, qbl_batched.hip: leading scalar kernel
# arguments arrive preloaded in registers at wave launch (the GEMV kernels'
# first loads then wait for no argument fetch); firmware without preloading
# runs the compiler's fallback prologue, which loads them.
EXTRA = {"qbl_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=9"],
         "qbl_batched.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=9"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
