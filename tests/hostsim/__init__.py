"""A CPU-only build of the library's host runtime for lifecycle tests.

The runtime source (quantized_base_linear_amd/csrc/qbl_runtime.cpp and
qbl_format.cpp, unchanged) is compiled with the host compiler against the HIP
test double in this directory (hip/hip_runtime.h, hip_sim.cpp): "device"
memory is tracked host memory and every kernel launch fails.  The result
exports the same C ABI, so the lifecycle calls (load, verify, budget, attach,
rollback, digests, fault injection) run here without a GPU, while every run
call reports QBL_E_DEVICE.  Test infrastructure only: the product library is
never built this way.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "quantized_base_linear_amd", "csrc")
SOURCES = [os.path.join(CSRC, "qbl_runtime.cpp"), os.path.join(CSRC, "qbl_format.cpp"),
           os.path.join(HERE, "hip_sim.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("qbl_host.h", "qbl_kernels.h")] + [
    os.path.join(ROOT, "include", "qbl.h"), os.path.join(HERE, "hip", "hip_runtime.h"),
    os.path.join(HERE, "hip", "hip_ext.h")]


def _compiler() -> str:
    # The runtime uses _Float16 on the host, which g++ 11 lacks; clang has it.
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("no clang++ to build the host-only test library")


def build() -> str:
    """Path of the host-only library, rebuilt when a source or header changes."""
    h = hashlib.sha256()
    for p in SOURCES + HEADERS:
        h.update(open(p, "rb").read())
    out_dir = os.path.join(tempfile.gettempdir(), "qbl_hostsim")
    os.makedirs(out_dir, exist_ok=True)
    so = os.path.join(out_dir, f"libqbl_hostsim_{h.hexdigest()[:16]}.so")
    if not os.path.exists(so):
        tmp = so + f".tmp{os.getpid()}"
        subprocess.run([_compiler(), "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-pthread",
                        "-I", HERE, "-o", tmp] + SOURCES, check=True)
        os.replace(tmp, so)
    return so


def load():
    """(Library bound to the host-only build, its raw CDLL with the sim hooks declared)."""
    import quantized_base_linear_amd as q
    lib = q.Library(build())
    raw = lib._lib
    for name in ("qbl_sim_live_bytes", "qbl_sim_live_allocations", "qbl_sim_bad_calls",
                 "qbl_sim_last_allocation"):
        getattr(raw, name).restype = ctypes.c_int64 if name != "qbl_sim_last_allocation" else ctypes.c_void_p
        getattr(raw, name).argtypes = []
    raw.qbl_sim_set_capacity.restype = None
    raw.qbl_sim_set_capacity.argtypes = [ctypes.c_int64]
    raw.qbl_sim_poke.restype = ctypes.c_int
    raw.qbl_sim_poke.argtypes = [ctypes.c_void_p, ctypes.c_uint8]
    return lib, raw
