"""Seeded synthetic inputs (SplitMix64 counter stream + Box-Muller normals).

Shared by the oracle tests and the GPU library's tests and benchmark.  It
holds none of the method's arithmetic: it draws float32 normal variates for
weights, adapter factors and activations, nothing else.  The C core
(``synth.c``) is built with gcc into ``libsynth.so`` next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (gcc, -O2, pthreads)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O3", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra",
             os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        lib.synth_splitmix64_at.restype = ctypes.c_uint64
        lib.synth_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_seed_from_tag.restype = ctypes.c_uint64
        lib.synth_seed_from_tag.argtypes = [ctypes.c_char_p]
        lib.synth_uniform_f64.restype = ctypes.c_int
        lib.synth_uniform_f64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        lib.synth_normal_f32.restype = ctypes.c_int
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_double, ctypes.c_double,
                                         ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def splitmix64_at(seed: int, i: int) -> int:
    return int(_load().synth_splitmix64_at(seed, i))


def seed(tag: str) -> int:
    """Stream seed of a textual tag."""
    return int(_load().synth_seed_from_tag(tag.encode()))


def normal(tag, shape, mean: float = 0.0, std: float = 1.0, offset: int = 0,
           out: np.ndarray | None = None, nthreads: int = 0) -> np.ndarray:
    """float32 array of N(mean, std) draws of the stream named by ``tag``.

    ``std`` is a standard deviation.  ``offset`` skips that many draws of the
    stream, so a slice of a large tensor can be drawn alone.
    """
    s = seed(tag) if isinstance(tag, str) else int(tag)
    shape = tuple(int(v) for v in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    n = int(np.prod(shape)) if shape else 1
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    rc = _load().synth_normal_f32(s, int(offset), n, float(mean), float(std),
                                  out.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError("synth_normal_f32 failed")
    return out


def uniform(tag, shape, offset: int = 0) -> np.ndarray:
    """float64 array of uniform [0, 1) draws (53-bit) of the stream named by ``tag``."""
    s = seed(tag) if isinstance(tag, str) else int(tag)
    shape = tuple(int(v) for v in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    out = np.empty(shape, dtype=np.float64)
    if _load().synth_uniform_f64(s, int(offset), out.size, out.ctypes.data) != 0:
        raise RuntimeError("synth_uniform_f64 failed")
    return out
